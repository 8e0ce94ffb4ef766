// Device helpers shared by the forward and backward kernels (internal to the library; not part of
// the C interface). gfx950 (CDNA4) only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa_detail {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kXcds = 8;  // MI355X: workgroups are dealt round-robin to 8 XCDs
constexpr int kMaxListTiles = 1024;  // block-sparse work lists: 64-row or 64-key tiles (per chunk)

template <bool BF16>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
    if constexpr (BF16) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                        __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                       __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
}

// Two fp32 values -> one packed pair, each rounded to nearest even.
template <bool BF16>
__device__ __forceinline__ unsigned pack2(float lo, float hi) {
    if constexpr (BF16) {
        bf16x2 v = {(__bf16)lo, (__bf16)hi};
        return __builtin_bit_cast(unsigned, v);
    } else {
        f16x2 v = {(_Float16)lo, (_Float16)hi};
        return __builtin_bit_cast(unsigned, v);
    }
}

// acc + lo + hi of a packed pair (the rounded probabilities, so the denominator sums exactly
// the weights the second product uses).
template <bool BF16>
__device__ __forceinline__ float add_pair(unsigned packed, float acc) {
    if constexpr (BF16) {
        const bf16x2 one = {(__bf16)1.f, (__bf16)1.f};
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, packed), one, acc, false);
    } else {
        const f16x2 one = {(_Float16)1.f, (_Float16)1.f};
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, packed), one, acc, false);
    }
}

// Value held by the lane 32 positions away (same query row, other half of the keys).
// (IEEE maximum, v_maximum3_f32: unlike fmaxf it needs no quieting of the swapped-in operands,
// which the compiler cannot see to be canonical; the scores it is used on are never NaN.)
__device__ __forceinline__ float fmax_ieee(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float max_with_partner(float x) {
    unsigned u = __float_as_uint(x);
    auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return fmax_ieee(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_with_partner(float x) {
    unsigned u = __float_as_uint(x);
    auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Workgroup -> (head, query tile). Workgroups are dealt to XCDs round-robin, so block b runs on
// XCD b % 8. Non-causal: give each XCD a contiguous range of (head, tile) pairs, so the
// workgroups resident on one XCD at a time share one head's K/V in that XCD's L2. Causal: each
// XCD owns whole heads and starts with their longest query tiles (most keys) so the short ones
// fill in at the end.
__device__ __forceinline__ void map_block(int bid, int G, int n_qt, bool causal, int& bh, int& qt) {
    if (G % kXcds == 0) {
        const int per = G / kXcds;
        const int x = bid % kXcds, s = bid / kXcds;
        if (!causal) {
            const int w = x * per + s;
            bh = w / n_qt;
            qt = w % n_qt;
            return;
        }
        if (per % n_qt == 0) {
            const int hpx = per / n_qt;
            qt = n_qt - 1 - s / hpx;
            bh = x * hpx + s % hpx;
            return;
        }
    }
    bh = bid / n_qt;
    qt = causal ? n_qt - 1 - bid % n_qt : bid % n_qt;
}

// 16x16x32 product: lane l holds row l % 16 of A and column l % 16 of B at k = 8(l / 16) .. +7,
// and C rows 4(l / 16) .. +3 of column l % 16. On random operands it sustains about 13% more
// flop/s than the 32x32x16 form under the power limit (same flops, less energy per flop).
template <bool BF16>
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
    if constexpr (BF16) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                        __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                       __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
}

// Max and sum over the four 16-lane rows of a wave (lanes l, l ^ 16, l ^ 32, l ^ 48): the lanes
// that hold one column of a 16x16 C tile.
__device__ __forceinline__ float max_over_rows(float x) {
    unsigned u = __float_as_uint(x);
    auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    u = __float_as_uint(fmax_ieee(__uint_as_float(a[0]), __uint_as_float(a[1])));
    auto b = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return fmax_ieee(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_over_rows(float x) {
    unsigned u = __float_as_uint(x);
    auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    u = __float_as_uint(__uint_as_float(a[0]) + __uint_as_float(a[1]));
    auto b = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// K and V tiles live in LDS as kBlockN rows of D elements (no padding); the 16-byte chunk c of
// row r is stored at chunk position c ^ swz(r). Both read patterns are then free of bank
// conflicts: the K operand reads one chunk from each of 16 consecutive rows, and the V^T
// transpose read takes 4 consecutive chunks from each of 4 consecutive rows.
template <int D>
__device__ __forceinline__ int swz(int r) {
    if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);  // 16 chunks per row
    else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);              // 8 chunks per row
}
template <int D>
__device__ __forceinline__ int tile_off(int r, int c) {  // element offset of (row, chunk)
    return r * D + ((c ^ swz<D>(r)) << 3);
}
// The forward kernel's 16x16x32 operands read their tiles in other patterns, with swizzles of
// their own (chosen by measured LDS read rates; each reaches the conflict-free rate):
// - K (swz_k): each 16-lane group reads one chunk from each of 16 consecutive rows, the four
//   groups chunks t, t + DT, t + 2DT, t + 3DT of the row (DT = D / 32);
// - V (swz_v): the transpose read takes two adjacent chunks (2b, 2b + 1) from each of 16
//   consecutive rows, and swz_v gives each 8 consecutive rows (for D = 64, whose rows are half
//   a bank line, each 8 rows of one parity) distinct chunk pairs.
template <int D>
__device__ __forceinline__ int swz_k(int r) {
    if constexpr (D == 128) return swz<128>(r);
    else return ((r & 3) << 1) | ((r >> 2) & 1);
}
template <int D>
__device__ __forceinline__ int tile_off_k(int r, int c) {
    return r * D + ((c ^ swz_k<D>(r)) << 3);
}
template <int D>
__device__ __forceinline__ int swz_v(int r) {
    if constexpr (D == 128) return ((r & 7) << 1) | ((r >> 3) & 1);  // 16 chunks per row
    else return (((r >> 1) & 3) << 1) | ((r >> 3) & 1);             // 8 chunks per row
}
template <int D>
__device__ __forceinline__ int tile_off_v(int r, int c) {
    return r * D + ((c ^ swz_v<D>(r)) << 3);
}

// Host: do two byte ranges overlap?
inline bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

// 16 bytes at byte offset `off` of the n_bytes at `head` into LDS, lane l's at dst + 16 l
// (buffer_load_dwordx4 ... lds). Offsets past n_bytes read zero (the buffer's range check; no
// memory beyond them is touched): the forward kernels pass a base at the tile's first row and the
// bytes up to the head's end, so rows past the sequence read as zero; the backward kernels clamp
// their rows instead. This is the MUBUF form of the LDS DMA on purpose: the compiler's wait-count pass
// takes the FLAT-encoded global_load_lds for an access that may touch LDS and finish out of
// order, and while one is in flight it waits for every LDS read (lgkmcnt(0)), also for those a
// register ring issued ahead; the MUBUF form counts only against vmcnt and leaves those waits
// exact. (The fourth descriptor word is gfx9's plain byte-addressed setting.)
__device__ __forceinline__ void lds_load16(const uint16_t* head, int n_bytes, unsigned off, lds_void* dst) {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)head, (short)0, n_bytes, 0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, off, 0, 0, 0);
}

// Block-sparse work lists. Of the tiles t0 .. t0 + T - 1, those that some wave of the workgroup
// needs (need(w, t) for wave w and absolute tile t) are compacted in ascending order into list
// (absolute tile index), with a byte per entry holding one bit per wave in wm. A ballot per wave
// and a prefix over the waves (through cnt[waves]) give each needed tile its position. Every
// thread of the workgroup calls it (it holds barriers); returns the number of entries, which is
// workgroup-uniform. With no entry, list[0] = t0 so that loads issued for entry 0 stay in range.
// The caller bounds T by the list's capacity.
template <int kWaves, typename Need>
__device__ __forceinline__ int compact_tiles(int t0, int T, Need need, int* list, uint8_t* wm, int* cnt, int tid) {
    constexpr int kThreads = 64 * kWaves;
    const int lane = tid & 63, wave = tid >> 6;
    int count = 0;
    for (int base = 0; base < T; base += kThreads) {
        const int t = base + tid;
        unsigned bits = 0;
        if (t < T) {
#pragma unroll
            for (int w = 0; w < kWaves; ++w)
                if (need(w, t0 + t)) bits |= 1u << w;
        }
        const uint64_t any = __builtin_amdgcn_ballot_w64(bits != 0);
        if (lane == 0) cnt[wave] = __builtin_popcountll(any);
        __syncthreads();
        int before = count, total = count;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const int cw = cnt[w];
            before += w < wave ? cw : 0;
            total += cw;
        }
        if (bits != 0) {
            const int pos = before + __builtin_popcountll(any & ((1ull << lane) - 1ull));
            list[pos] = t0 + t;
            wm[pos] = (uint8_t)bits;
        }
        count = total;
        __syncthreads();
    }
    if (count == 0) {
        if (tid == 0) list[0] = t0;
        __syncthreads();
    }
    return count;
}

}  // namespace fa_detail
