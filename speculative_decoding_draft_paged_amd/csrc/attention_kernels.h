// gfx950 kernels for draft-block paged attention (templates; instantiated per KV element type by
// kernels_bf16.hip and kernels_fp8.hip).
//
// Attention kernels (split-KV attention and its epilogue). One workgroup = one
// work unit: a range of 32-token key tiles of one (request b, kv head). Per tile:
//   - S^T = K Q^T on v_mfma_f32_16x16x32_bf16. Tokens are the M dimension and
//     the query rows the N dimension, so every lane owns one query row of S^T
//     and the softmax statistics stay in-lane (four lanes per row: one quad each);
//   - online softmax in exp2 space (scores pre-multiplied by sm_scale*log2 e),
//     masks only on edge tiles; V rows past the sequence end are zeroed by
//     select, so stale cache slots (even NaN) cannot leak through 0 * NaN;
//   - O^T += V^T P^T on the same MFMA with P rounded to bf16; the P operand is
//     exactly the lane's own S^T accumulator registers (no shuffles). V^T comes
//     from a row-major V tile in LDS through the transposing LDS read.
// Windowed form: row i's keys are its causal window (p - W, p] and the block keys
// after it, (p, min(N - 1, p + W_r)], all inside the unit's tiles. The block keys
// after a query are folded into the running softmax state by the online update,
// which is the log-sum-exp merge of TensorRT-LLM PR #21130 (Description item 1 and
// its formulation table: lse = lse_c (+) lse_f with out weighted by 2^(lse_c - lse)
// and 2^(lse_f - lse)) applied tile by tile; with K = 1 or W_r = 0 no later key
// exists and the causal result is returned as is (item 2).
//
// stream_kernel (R <= 32): one row-wave, WT token groups per workgroup streaming
// interleaved tiles, no workgroup barrier in the loop. K goes straight from HBM
// into the MFMA A fragments; V goes row-major into a private LDS tile. Two tiles
// are in flight per wave, and the page ids of up to 2048 tiles are staged in LDS
// once per window, so no scalar load sits on the path.
// shared_kernel (R > 32): several row-waves consume every tile from an LDS ring
// the whole workgroup fills (see there).
// Epilogue: the token groups of the workgroup merge through LDS. A unit that is
// its request's only split writes the final bf16 output and base-2 LSE itself;
// otherwise it writes its fp32 (acc, m, l) partial.
//
// combine_kernel: the LSE combine of the splits, several output rows per workgroup,
// launched after the attention kernel. (Combining inside the attention kernel by
// its last-finishing unit needs an agent-scope release and acquire per unit; on
// this part those cache write-backs cost far more than a second launch.)
//
// The split-KV form itself follows TensorRT-LLM PR #16150 (paged DFlash
// cross-attention; its commit list reworks the kernel flash-decoding style and
// makes the split count a runtime argument) and the multi-CTA split-KV of
// PR #20374, redone for 64-wide wavefronts, MFMA tiles and HND pages.
#pragma once

#include "internal.h"

#include <math.h>

#include <atomic>
#include <type_traits>

namespace blockattn {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));

constexpr float kNegInf = -__builtin_huge_valf();
constexpr int T = kTileTokens;
template <int D>
constexpr int kLog2 = D == 64 ? 6 : 7;

// LDS row pitches (bf16 elements) of staged K and V tiles. Both reads of a tile
// move 256 bytes per cycle: the K fragment read (16 bytes per lane; lanes of eight
// rows in two column groups served together) and the transposing V read (8 bytes
// per lane; eight rows of 32 bytes together). Measured on gfx950, a row stride of 32
// modulo 256 bytes is free of bank conflicts for both (16, 48, 64 or 80 give
// two-way conflicts, 0 eight-way), and the rule only needs an odd multiple of 32
// bytes, which D + 16 elements gives for D = 64 (160 bytes) and 128 (288 bytes).
template <int D>
constexpr int kKPitch = D + 16;
template <int D>
constexpr int kVPitch = D + 16;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// fp32 -> bf16 by round-to-nearest-even. Carrying into the exponent field rounds a magnitude at
// or past the midpoint between the largest finite bf16 and 2^128 to infinity; every NaN becomes
// the canonical quiet NaN 0x7FC0.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)0x7FC0u;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

// Record an input that had to be clamped (a device length or a page id out of range) in the
// workspace's input-error word. The clamp keeps every read inside the caller's buffers; the
// word lets a caller find out that the result is not the one its inputs describe.
__device__ __forceinline__ void flag_input_error(uint32_t* err, uint32_t bits) {
    __hip_atomic_fetch_or(err, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Profiling aid: when the caller gave a trace buffer, the workgroup's first lane writes the
// constant 100 MHz clock for phase `k` of this unit, after every memory operation the wave has in
// flight has completed (so a phase ends when its data has arrived). Off (one uniform branch) when
// no buffer is given.
__device__ __forceinline__ void trace_point(const KernelArgs& a, int k) {
    if (a.trace != nullptr) {
        __builtin_amdgcn_s_waitcnt(0);
        const uint64_t t = __builtin_amdgcn_s_memrealtime();
        if (threadIdx.x == 0) a.trace[(size_t)blockIdx.x * kTracePoints + k] = t;
    }
}

// Page id entry `v` of a page-table row, clamped into [0, num_pages).
__device__ __forceinline__ int checked_page(const KernelArgs& a, int v) {
    if ((unsigned)v >= (unsigned)a.num_pages) {
        flag_input_error(a.err, kErrPage);
        v = clampi(v, 0, a.num_pages - 1);
    }
    return v;
}

__device__ __forceinline__ u32x4_t ldg16(const uint16_t* p) { return *(const u32x4_t*)p; }

// Sixteen bytes of a pool starting at element `e`: 8 bf16 or 16 fp8 E4M3 elements.
template <bool FP8>
__device__ __forceinline__ u32x4_t ldkv16(const void* pool, size_t e) {
    return __builtin_nontemporal_load((const u32x4_t*)(static_cast<const char*>(pool) + e * (FP8 ? 1 : 2)));
}

// OCP E4M3 of an fp32 value by round-to-nearest-even, saturating at +-448; NaN -> 0x7F.
__device__ __forceinline__ uint32_t f32_to_e4m3_sat(float q) {
    const uint32_t u = __float_as_uint(q);
    const uint32_t sign = (u >> 24) & 0x80u;
    const float a = fabsf(q);
    if (a != a) return 0x7Fu;
    if (a >= 448.f) return sign | 0x7Eu;
    if (a < 0.015625f) return sign | (uint32_t)__builtin_rintf(a * 512.f);  // below 2^-6: multiples of 2^-9
    int e = (int)((u >> 23) & 0xFFu) - 127;                                 // -6 .. 8
    uint32_t m3 = (u >> 20) & 7u;
    const uint32_t rem = u & 0xFFFFFu;
    if (rem > 0x80000u || (rem == 0x80000u && (m3 & 1u))) ++m3;
    if (m3 == 8u) {
        m3 = 0;
        ++e;
    }
    if (e > 8 || (e == 8 && m3 == 7u)) return sign | 0x7Eu;
    return sign | ((uint32_t)(e + 7) << 3) | m3;
}

// Eight elements as bf16 (exact: every E4M3 value is a bf16 value).
__device__ __forceinline__ u32x4_t widen8(u32x4_t v) { return v; }
__device__ __forceinline__ u32x4_t widen8(u32x2_t v) {
    const auto c0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.x, 1.0f, false);
    const auto c1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.x, 1.0f, true);
    const auto c2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.y, 1.0f, false);
    const auto c3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.y, 1.0f, true);
    return u32x4_t{__builtin_bit_cast(uint32_t, c0), __builtin_bit_cast(uint32_t, c1), __builtin_bit_cast(uint32_t, c2),
                   __builtin_bit_cast(uint32_t, c3)};
}

// Transposing LDS read (ds_read_b64_tr_b16). Within each 16-lane group, lane l
// receives element l % 4 of the 8 bytes addressed by lane 4e + (l % 16) / 4, for
// e = 0..3. With lane l pointing at row l/4, columns 4(l%4)..+3 of a row-major
// 4 x 16 block, lane l gets column l of that block (4 rows).
__device__ __forceinline__ u32x2_t lds_read_tr16(const uint16_t* p) {
    i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)(p));
    return __builtin_bit_cast(u32x2_t, v);
}

// Maximum over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (the four quads holding one
// row's tokens), with the gfx950 row-swap permutes: swapping 16-lane rows between
// two copies of x pairs rows (0,1) and (2,3), swapping 32-lane halves pairs (0,2)
// and (1,3). VALU only, so no LDS round trip sits in the softmax chain.
__device__ __forceinline__ float quad_max(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const float m = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Sum over the same four lanes; every lane gets the same bits ((x0 + x1) + (x2 + x3)
// in a lane-independent order).
__device__ __forceinline__ float quad_sum(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const float m = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// First of the 8 contraction elements that lane quad `quad` holds for K-step kk of a
// 32-element MFMA step: 32 kk + 8 quad in order, or with `pair` 64 (kk / 2) + 16 quad +
// 8 (kk % 2), so one 16-byte fp8 load of 16 consecutive elements feeds two steps.
template <bool pair>
__device__ __forceinline__ int kelem(int kk, int quad) {
    return pair ? 64 * (kk >> 1) + 16 * quad + 8 * (kk & 1) : 32 * kk + 8 * quad;
}

// N keys, the last K of them the block (p = C + i); NC of them are read from the
// cache (N, or C when the block comes from dense arrays); tiles [ulo, uhi).
struct Unit {
    int b, hk, rg, s, S, N, C, NC, ulo, uhi;  // rg: row group (rows rg * R .. of the kv head)
};

template <bool WINDOWED>
__device__ __forceinline__ Unit decode_unit(const KernelArgs& a) {
    WorkItem wi;
    const int hv_count = a.Hkv * a.row_groups;  // (kv head, row group) pairs per request
    if (a.uniform_splits > 0) {  // every pair has the same split count: no work-list load
        const int pair = blockIdx.x / a.uniform_splits;
        wi.b = pair / hv_count;
        wi.hk = pair - wi.b * hv_count;
        wi.s = blockIdx.x - pair * a.uniform_splits;
        wi.S = a.uniform_splits;
    } else {
        wi = a.work[blockIdx.x];
    }
    Unit u;
    u.b = wi.b;
    u.hk = wi.hk / a.row_groups;
    u.rg = wi.hk - u.hk * a.row_groups;
    u.s = wi.s;
    u.S = wi.S;
    const int n_dev = a.seq_lens[wi.b];
    u.N = clampi(n_dev, a.K, a.stride * a.P);
    if (u.N != n_dev && threadIdx.x == 0) flag_input_error(a.err, kErrLength);
    u.C = u.N - a.K;
    u.NC = a.k_block ? u.C : u.N;
    const int key_lo = (WINDOWED && a.window_left > 0) ? max(0, u.C - a.window_left + 1) : 0;
    const int tb = key_lo / T, te = max(tb, (u.NC + T - 1) / T), nt = te - tb;
    u.ulo = tb + (int)((int64_t)wi.s * nt / wi.S);
    u.uhi = tb + (int)((int64_t)(wi.s + 1) * nt / wi.S);
    return u;
}

// Per-wave query fragments (B operand of S^T = K Q^T), row key bounds and softmax state.
// ALL_ON: every owned 16-row block holds live rows (no per-block skip test).
template <int D, int NBW, bool WINDOWED, bool ALL_ON = false>
struct WaveRows {
    static constexpr int KK = D / 32, DB = D / 16;
    bf16x8_t qf[NBW][KK];
    int row_lo[NBW], row_hi[NBW];
    bool on[NBW];
    f32x4_t acc[NBW][DB];
    float m[NBW], l[NBW];
    float neg_m[NBW];  // -m, or 0 while m = -inf
    float gate[NBW];   // exponent arguments above this need the slow path: -inf before a row's first key
                       // (so any key sets m), the rescale slack after
    int lo_max, hi_min;
    int hi_cap;  // keys at or past this come from elsewhere (the dense block) and are masked here

    // kpair: the contraction elements of K-steps 2h and 2h + 1 are taken as lane quad's
    // 16 consecutive elements 64h + 16 quad .. + 15 (first 8 to step 2h), so that one
    // 16-byte load of 16 fp8 keys feeds two steps; the keys use the same layout. A dot
    // product does not depend on the order of its terms, only on Q and K agreeing.
    template <bool kpair = false>
    __device__ __forceinline__ void init(const KernelArgs& a, const Unit& u, int first_block, int lane) {
        const int r16 = lane & 15, quad = lane >> 4;
        const bool left_win = WINDOWED && a.window_left > 0;
        const int right = a.window_right < 0 ? a.K : a.window_right;  // later block keys a row sees
#pragma unroll
        for (int n = 0; n < NBW; ++n) {
            const int nb = first_block + n;
            const int r0 = u.rg * a.R + nb * 16;  // first row of the block in the kv head's R_all rows
            const int r = r0 + r16;
            on[n] = nb * 16 < a.R && r0 < a.R_all;
            const bool live = nb * 16 + r16 < a.R && r < a.R_all;
            const int i = live ? r / a.g : a.K - 1;
            const int lg = live ? r - (r / a.g) * a.g : 0;
            const uint16_t* qrow = a.q + ((size_t)(u.b * a.K + i) * a.Hq + u.hk * a.g + lg) * D;
#pragma unroll
            for (int kk = 0; kk < KK; ++kk)
                qf[n][kk] = __builtin_bit_cast(bf16x8_t, live ? ldg16(qrow + kelem<kpair>(kk, quad))
                                                              : u32x4_t{0u, 0u, 0u, 0u});
            const int p = u.C + i;
            row_lo[n] = left_win ? max(0, p - a.window_left + 1) : 0;
            // windowed: the causal window and the block keys after the query up to p + W_r
            row_hi[n] = WINDOWED ? min(u.N - 1, p + right) : u.N - 1;
            m[n] = kNegInf;
            l[n] = 0.f;
            neg_m[n] = 0.f;
            gate[n] = kNegInf;
#pragma unroll
            for (int db = 0; db < DB; ++db) acc[n][db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
        lo_max = left_win ? max(0, u.C + a.K - a.window_left) : 0;
        hi_min = WINDOWED ? min(u.N - 1, u.C + right) : u.N - 1;
        hi_cap = u.NC;
    }

    // Scores of one tile for every owned row block. ALL: also for a block with no live
    // rows (zero queries; its state is never stored), so the code has no branch.
    template <bool ALL = false>
    __device__ __forceinline__ void scores(const bf16x8_t (&kf)[2][KK], f32x4_t (&s)[NBW][2]) const {
#pragma unroll
        for (int n = 0; n < NBW; ++n) {
            s[n][0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            s[n][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            if (ALL_ON || ALL || on[n]) {
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
                    for (int mb = 0; mb < 2; ++mb)
                        s[n][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[mb][kk], qf[n][kk], s[n][mb], 0, 0, 0);
                }
            }
        }
    }

    // Online softmax update and O^T += V^T P^T for one tile starting at token t0, in
    // two parts: prep (masking, exponent arguments, the rare move of the reference)
    // and apply (probabilities, row sums and the PV product), so a caller can issue
    // other work between them.
    // m[n] is the reference maximum (log2 units) the row sums are kept relative to.
    // It only moves when a score exceeds it by more than kRescaleSlack, so the
    // accumulator rescale is rare and probabilities stay below 2^kRescaleSlack
    // (exact in fp32 and representable in bf16). The softmax scale is folded into
    // the exponent's FMA.
    // The scores are masked in place (s is consumed).
    template <bool ALL = false>
    __device__ __forceinline__ void prep(f32x4_t (&s)[NBW][2], int t0, float scale, int quad, float (&y)[NBW][8]) {
        constexpr float kRescaleSlack = 8.f;
        const bool edge = (t0 < lo_max) || (t0 + T - 1 > hi_min) || (t0 + T > hi_cap);
#pragma unroll
        for (int n = 0; n < NBW; ++n) {
            if (!ALL_ON && !ALL && !on[n]) continue;
            if (__builtin_expect(edge, 0)) {  // a tile at the window's edges (rare): mask in place
                const int lo = row_lo[n], hi = min(row_hi[n], hi_cap - 1);
#pragma unroll
                for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int tok = t0 + mb * 16 + quad * 4 + j;
                        s[n][mb][j] = (tok < lo || tok > hi) ? kNegInf : s[n][mb][j];
                    }
            }
            float x[8];
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int j = 0; j < 4; ++j) x[mb * 4 + j] = s[n][mb][j];
            // Exponent arguments against the current reference. They are arithmetic
            // results, so their maximum needs no operand canonicalisation. The row's
            // four-lane maximum is needed only when an argument passes the gate; a row's
            // maximum is at least each of its lanes' maxima, so when no lane of the wave
            // passes (the common case after a row's first tile) no row needs a rescale.
#pragma unroll
            for (int k = 0; k < 8; ++k) y[n][k] = fmaf(x[k], scale, neg_m[n]);
            const float ymax = fmaxf(fmaxf(fmaxf(y[n][0], y[n][1]), fmaxf(y[n][2], y[n][3])),
                                     fmaxf(fmaxf(y[n][4], y[n][5]), fmaxf(y[n][6], y[n][7])));
            if (__builtin_amdgcn_ballot_w64(ymax > gate[n]) != 0) {
                const float mx = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
                const float mxs = quad_max(mx) * scale;  // scale > 0, so the maximum commutes with it
                if (mxs > m[n] + kRescaleSlack) {
                    const float alpha = fast_exp2(m[n] - mxs);
                    l[n] *= alpha;
#pragma unroll
                    for (int db = 0; db < DB; ++db) acc[n][db] *= alpha;
                    m[n] = mxs;
                    neg_m[n] = -mxs;
                    gate[n] = kRescaleSlack;
                }
#pragma unroll
                for (int k = 0; k < 8; ++k) y[n][k] = fmaf(x[k], scale, neg_m[n]);
            }
        }
    }

    // PMUL: the tile's values are in other units than the accumulator's; each
    // probability is multiplied by pmul (after it joins the row sum) before its bf16
    // rounding for the P V product.
    template <bool PMUL = false, bool ALL = false>
    __device__ __forceinline__ void apply(const float (&y)[NBW][8], const bf16x8_t (&vf)[DB], float pmul = 1.f) {
#pragma unroll
        for (int n = 0; n < NBW; ++n) {
            if (!ALL_ON && !ALL && !on[n]) continue;
            bf16x8_t pb;
            float p[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                p[k] = fast_exp2(y[n][k]);
                if constexpr (PMUL)
                    pb[k] = (__bf16)(p[k] * pmul);
                else
                    pb[k] = (__bf16)p[k];
            }
            l[n] += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
#pragma unroll
            for (int db = 0; db < DB; ++db)
                acc[n][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[db], pb, acc[n][db], 0, 0, 0);
        }
    }

    template <bool PMUL = false>
    __device__ __forceinline__ void update(f32x4_t (&s)[NBW][2], const bf16x8_t (&vf)[DB], int t0, float scale,
                                           int quad, float pmul = 1.f) {
        float y[NBW][8];
        prep(s, t0, scale, quad, y);
        apply<PMUL>(y, vf, pmul);
    }
};

// Floats of LDS the epilogue needs (it reuses the tile buffers): per token group
// and row the (m, l) pair, and the scaled accumulators of token groups 1..WT-1
// (row pitch D + 8 floats: an odd multiple of 32 bytes, free of bank conflicts).
__host__ __device__ constexpr size_t epilogue_floats(int D, int slots_per_group, int token_groups) {
    return token_groups <= 1 ? 0
                             : (size_t)token_groups * slots_per_group * 16 * 2 +
                                   (size_t)(token_groups - 1) * slots_per_group * 16 * (D + 8);
}

// Device-scope accesses for the split partials when the last split of a (request, kv head)
// combines them inside the attention kernel. The stores write through to where every compute
// unit's loads see them once they complete, and the loads read there, so the hand-off needs no
// cache-wide release or acquire (an L2 write-back or invalidate): only each storing wave's wait
// for its stores to complete before the arrival counter moves.
__device__ __forceinline__ void st_dev(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev4(float* p, f32x4_t v) {
    uint64_t* q = reinterpret_cast<uint64_t*>(p);
    __hip_atomic_store(q, (uint64_t)__float_as_uint(v[0]) | ((uint64_t)__float_as_uint(v[1]) << 32), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(q + 1, (uint64_t)__float_as_uint(v[2]) | ((uint64_t)__float_as_uint(v[3]) << 32),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float* p) {
    return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Sixteen bytes at byte offset `off` of a buffer, read at device scope (the sc1 cache policy).
constexpr int kCachePolicyDevice = 16;
constexpr int kCachePolicyStream = 2;  // non-temporal: each byte of the pools is read once per call
__device__ __forceinline__ f32x4_t ld_dev4(__amdgpu_buffer_rsrc_t buf, uint32_t off) {
    return __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(buf, off, 0, kCachePolicyDevice));
}
// Raw buffer resource over `bytes` bytes at p (gfx9 descriptor word 3 for untyped dword access).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// Store one wave's rows: acc holds O^T fragments (lane: query row r16 of block n,
// dims db*16 + 4*quad .. +3), already scaled to the row's final weights when
// `final`, else relative to 2^m. m, l: the row's reference maximum (log2 units)
// and weight sum. dev: partials go out with device-scope stores (combined in-kernel).
template <int D>
__device__ __forceinline__ void store_rows(const KernelArgs& a, const Unit& u, int r, bool final, const f32x4_t (&acc)[D / 16],
                                           float m, float l, int quad, bool dev) {
    constexpr int DB = D / 16;
    if (r >= a.R || u.rg * a.R + r >= a.R_all) return;
    f32x4_t acc_s[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) acc_s[db] = acc[db] * a.v_scale;  // a stored value stands for v_scale * v
    if (!final) {
        const size_t pr = (size_t)blockIdx.x * a.R + r;
        if (dev) {
#pragma unroll
            for (int db = 0; db < DB; ++db) st_dev4(a.part_acc + pr * D + db * 16 + quad * 4, acc_s[db]);
            if (quad == 0) {
                st_dev(a.part_m + pr, m);
                st_dev(a.part_l + pr, l);
            }
        } else {
#pragma unroll
            for (int db = 0; db < DB; ++db) *(f32x4_t*)(a.part_acc + pr * D + db * 16 + quad * 4) = acc_s[db];
            if (quad == 0) {
                a.part_m[pr] = m;
                a.part_l[pr] = l;
            }
        }
        return;
    }
    const int rk = u.rg * a.R + r;  // row in the kv head's R_all rows
    const int i = rk / a.g, h = u.hk * a.g + (rk - (rk / a.g) * a.g);
    const size_t orow = (size_t)(u.b * a.K + i) * a.Hq + h;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        const uint32_t lo = f32_to_bf16_rne(acc_s[db][0]) | ((uint32_t)f32_to_bf16_rne(acc_s[db][1]) << 16);
        const uint32_t hi = f32_to_bf16_rne(acc_s[db][2]) | ((uint32_t)f32_to_bf16_rne(acc_s[db][3]) << 16);
        *(u32x2_t*)(a.out + orow * D + db * 16 + quad * 4) = u32x2_t{lo, hi};
    }
    if (quad == 0 && a.lse) a.lse[orow] = l == 0.f ? kNegInf : m + log2f(l);  // a NaN sum stays NaN
}

// The split combine inside the attention kernel, by the last unit of a (request, kv head,
// row group) to finish (the multi-CTA split-KV of TensorRT-LLM PR #20374, Description: the
// splits of a decode row meet through counter buffers). Every unit of a split pair has
// stored its partial with device-scope stores; each storing wave waits for them to complete,
// then one thread adds 1 to the pair's arrival counter. The unit that brings the counter to
// S resets it for the next call and combines the S partials in split order: per row
// M = max m_s, L = sum 2^(m_s - M) l_s, out = sum 2^(m_s - M) acc_s / L, lse = M + log2 L. An
// empty split (m = -inf) weighs 0; 0 * NaN still carries a NaN sum through. No unit waits for
// another: the last arriver only reads what has already completed.
template <int D>
__device__ void combine_if_last(const KernelArgs& a, const Unit& u, float* lds) {
    constexpr int DL = D / 4;  // float4 columns of a row
    const int tid = threadIdx.x, nt = blockDim.x;
    const int S = u.S, R = a.R;
    __builtin_amdgcn_s_waitcnt(0);  // this wave's partial stores have completed
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __syncthreads();  // every wave's have; the epilogue is done with LDS
    int* flag = reinterpret_cast<int*>(lds);
    if (tid == 0) {
        const int pair = (u.b * a.Hkv + u.hk) * a.row_groups + u.rg;
        const uint32_t old = __hip_atomic_fetch_add(a.counters + pair, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int last = old == (uint32_t)(S - 1);
        if (last) __hip_atomic_store(a.counters + pair, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *flag = last;
    }
    __syncthreads();
    if (*flag == 0) return;
    __atomic_signal_fence(__ATOMIC_SEQ_CST);

    const int u0 = blockIdx.x - u.s;  // the pair's units are consecutive
    // One item per float4 column of a row. Each item folds the pair's S partials in split
    // order into a running (m, l, acc) state, as the combine kernel does, so all of its loads
    // are independent and issue together: one round trip from the last unit's arrival to its
    // output. The partials are S consecutive [R] (m, l) and [R][D] (acc) blocks.
    const __amdgpu_buffer_rsrc_t accs = make_rsrc(a.part_acc + (size_t)u0 * R * D, (uint32_t)((size_t)S * R * D * 4));
    const __amdgpu_buffer_rsrc_t mrs = make_rsrc(a.part_m + (size_t)u0 * R, (uint32_t)((size_t)S * R * 4));
    const __amdgpu_buffer_rsrc_t lrs = make_rsrc(a.part_l + (size_t)u0 * R, (uint32_t)((size_t)S * R * 4));
    for (int it = tid; it < R * DL; it += nt) {
        const int rr = it / DL, c = (it - (it / DL) * DL) * 4;
        const int rk = u.rg * R + rr;
        if (rk >= a.R_all) continue;
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
        float m = kNegInf, l = 0.f;
        const uint32_t abase = (uint32_t)((rr * D + c) * 4), astep = (uint32_t)(R * D * 4);
#pragma unroll 8
        for (int s = 0; s < S; ++s) {
            const uint32_t so = (uint32_t)((s * R + rr) * 4);
            const float ms = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(mrs, so, 0, kCachePolicyDevice));
            const float ls = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(lrs, so, 0, kCachePolicyDevice));
            const f32x4_t as = ld_dev4(accs, abase + (uint32_t)s * astep);
            // a split with no keys (m = -inf) weighs 0; 0 * NaN still carries a NaN sum through
            const float mn = fmaxf(m, ms);
            const float wa = m == kNegInf ? 0.f : fast_exp2(m - mn);
            const float wb = ms == kNegInf ? 0.f : fast_exp2(ms - mn);
            acc = acc * wa + as * wb;
            l = l * wa + ls * wb;
            m = mn;
        }
        const float inv = l == 0.f ? 0.f : 1.f / l;  // no keys: zeros; a NaN sum stays NaN
        const f32x4_t o = acc * inv;
        const int i = rk / a.g, h = u.hk * a.g + (rk - (rk / a.g) * a.g);
        const size_t orow = (size_t)(u.b * a.K + i) * a.Hq + h;
        const uint32_t lo = f32_to_bf16_rne(o[0]) | ((uint32_t)f32_to_bf16_rne(o[1]) << 16);
        const uint32_t hi = f32_to_bf16_rne(o[2]) | ((uint32_t)f32_to_bf16_rne(o[3]) << 16);
        *(u32x2_t*)(a.out + orow * D + c) = u32x2_t{lo, hi};
        if (c == 0 && a.lse) a.lse[orow] = l == 0.f ? kNegInf : m + log2f(l);
    }
}

// Epilogue of a unit: merge the token groups' softmax states, then write the
// unit's partial (a split request) or the final bf16 output and base-2 LSE.
// With one token group every wave owns whole rows and stores from registers.
// Every wave of the workgroup runs to the end (the in-kernel combine has barriers).
template <int D, int NBW, bool WINDOWED, bool ALL_ON>
__device__ void finish_unit(const KernelArgs& a, const Unit& u, WaveRows<D, NBW, WINDOWED, ALL_ON>& w, int tg,
                            int wr, int WT, int WR, float* lds) {
    constexpr int DB = D / 16, XP = D + 8;
    const int tid = threadIdx.x;
    const int lane = tid & 63, r16 = lane & 15, quad = lane >> 4;
    const int slots = WR * NBW;  // row blocks per token group
    const bool final = u.S <= 1;
    const bool fused = !final && a.fused_combine;

#pragma unroll
    for (int n = 0; n < NBW; ++n) w.l[n] = quad_sum(w.l[n]);

    if (WT == 1) {
#pragma unroll
        for (int n = 0; n < NBW; ++n) {
            if (!ALL_ON && !w.on[n]) continue;
            const float l = w.l[n];
            const float inv = final ? (l == 0.f ? 0.f : 1.f / l) : 1.f;  // no keys: zeros; a NaN sum stays NaN
#pragma unroll
            for (int db = 0; db < DB; ++db) w.acc[n][db] *= inv;
            store_rows<D>(a, u, (wr * NBW + n) * 16 + r16, final, w.acc[n], w.m[n], l, quad, fused);
        }
    } else {
        float* ml = lds;                                   // [WT][slots * 16][2]
        float* xa = lds + (size_t)WT * slots * 16 * 2;     // [WT - 1][slots * 16][XP]
        __syncthreads();  // tile buffers are free from here on
        trace_point(a, kTrEpilogue);
#pragma unroll
        for (int n = 0; n < NBW; ++n)
            if (quad == 0) {
                float* e = ml + ((size_t)(tg * slots + wr * NBW + n) * 16 + r16) * 2;
                e[0] = w.m[n];
                e[1] = w.l[n];
            }
        __syncthreads();
        float rowM[NBW], rowL[NBW];
#pragma unroll
        for (int n = 0; n < NBW; ++n) {
            const int srow = (wr * NBW + n) * 16 + r16;
            float M = kNegInf;
            for (int t = 0; t < WT; ++t) M = fmaxf(M, ml[((size_t)t * slots * 16 + srow) * 2]);
            // A group with no keys (m = -inf) weighs 0; 0 * NaN still carries a NaN sum through.
            float L = 0.f;
            for (int t = 0; t < WT; ++t) {
                const float* e = ml + ((size_t)t * slots * 16 + srow) * 2;
                L += (e[0] == kNegInf ? 0.f : fast_exp2(e[0] - M)) * e[1];
            }
            float alpha = w.m[n] == kNegInf ? 0.f : fast_exp2(w.m[n] - M);
            if (final) alpha = L == 0.f ? 0.f : alpha / L;
#pragma unroll
            for (int db = 0; db < DB; ++db) w.acc[n][db] *= alpha;
            rowM[n] = M;
            rowL[n] = L;
            if (tg > 0) {
                float* x = xa + ((size_t)(tg - 1) * slots * 16 + srow) * XP;
#pragma unroll
                for (int db = 0; db < DB; ++db) *(f32x4_t*)(x + db * 16 + quad * 4) = w.acc[n][db];
            }
        }
        __syncthreads();
        if (tg == 0) {
#pragma unroll
            for (int n = 0; n < NBW; ++n) {
                if (!ALL_ON && !w.on[n]) continue;
                const int srow = (wr * NBW + n) * 16 + r16;
                for (int t = 1; t < WT; ++t) {
                    const float* x = xa + ((size_t)(t - 1) * slots * 16 + srow) * XP;
#pragma unroll
                    for (int db = 0; db < DB; ++db) w.acc[n][db] += *(const f32x4_t*)(x + db * 16 + quad * 4);
                }
                store_rows<D>(a, u, srow, final, w.acc[n], rowM[n], rowL[n], quad, fused);
            }
        }
    }
    if (a.trace) {
        __syncthreads();
        trace_point(a, kTrStored);
    }
    if (fused) combine_if_last<D>(a, u, lds);
}

// Store the block's keys and values (dense bf16 [B, K, Hkv, D]) of this unit's
// (b, h_kv) into their cache slots C .. C + K - 1, encoded for the pool: the fp32
// quotient by the pool scale, rounded to bf16 or to saturating E4M3.
template <int D, bool FP8>
__device__ void append_block(const KernelArgs& a, const Unit& u) {
    const int32_t* pt_row = a.page_table + (size_t)u.b * a.stride;
    const int pmask = (1 << a.p_shift) - 1;
    const int n = a.K * D;
    for (int idx = threadIdx.x; idx < 2 * n; idx += blockDim.x) {
        const bool isv = idx >= n;
        const int e = isv ? idx - n : idx;
        const int i = e / D, d = e - (e / D) * D;
        const int j = u.C + i;
        const int page = checked_page(a, pt_row[j >> a.p_shift]);
        const size_t off = (((size_t)page * a.Hkv + u.hk) << (a.p_shift + kLog2<D>)) + (size_t)(j & pmask) * D + d;
        const uint16_t xb = (isv ? a.v_block : a.k_block)[((size_t)(u.b * a.K + i) * a.Hkv + u.hk) * D + d];
        const float q = bf16_to_f32(xb) / (isv ? a.v_scale : a.k_scale);
        void* pool = const_cast<void*>(isv ? a.vc : a.kc);
        if constexpr (FP8)
            static_cast<uint8_t*>(pool)[off] = (uint8_t)f32_to_e4m3_sat(q);
        else
            static_cast<uint16_t*>(pool)[off] = f32_to_bf16_rne(q);
    }
}

// ---------------------------------------------------------------------------------
// Streaming main loop: one wave owns every row (R <= 16 * NBW), WT waves per
// workgroup stream interleaved tiles of the unit, two tiles in flight per wave.
// The page ids of up to kPidWindow tiles are staged in LDS by the whole workgroup
// (one gather round trip), so the tile loads depend only on short LDS reads. Every
// global load of the loop sits at a fixed, unconditional place, which keeps the
// compiler's wait counts exact: the wait for one tile never drains the tile behind
// it. The loop stops while a third tile still follows the pair in flight; the last
// one or two tiles are consumed after it with no further loads.
template <int D, int NBW, bool WINDOWED, bool ALL_ON, int MAXT, bool FP8>
__global__ __launch_bounds__(MAXT) void stream_kernel(const KernelArgs a) {
    constexpr int KK = D / 32, DB = D / 16;
    // Every K and V load is 16 bytes per lane: 8 bf16 elements, or 16 fp8 elements (the
    // keys then in the paired contraction layout, so one load feeds two K-steps).
    constexpr int KL = FP8 ? KK / 2 : KK;  // K loads per 16-row block
    constexpr int VE = FP8 ? 16 : 8;       // V elements per lane load
    constexpr int RPC = 64 * VE / D;       // tile rows per 1-KiB chunk (64 lanes x 16 bytes)
    constexpr int VCH = T / RPC;           // chunks of the 32-row V tile
    constexpr int VP = kVPitch<D>;         // padded row pitch of the V tile in LDS (bf16 elements)
    static_assert(VCH * RPC == T && 16 % RPC == 0, "V chunks cover the tile and never straddle its halves");

    extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
    const int tid = threadIdx.x, nthreads = blockDim.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar) index
    const int r16 = lane & 15, quad = lane >> 4;
    const int WT = a.token_groups, WR = a.row_waves;
    const int tg = wave / WR, wr = wave - (wave / WR) * WR;  // token group, row group
    trace_point(a, kTrEntry);
    const Unit u = decode_unit<WINDOWED>(a);
    trace_point(a, kTrLength);
    WaveRows<D, NBW, WINDOWED, ALL_ON> w;
    w.template init<FP8>(a, u, wr * NBW, lane);
    // LDS: [one V tile per wave] [page-id window]
    uint16_t* vlds = lds + (size_t)wave * T * VP;
    int* pid_tab = reinterpret_cast<int*>(lds + (size_t)WT * WR * T * VP);

    const int32_t* pt_row = a.page_table + (size_t)u.b * a.stride;
    const int last_page = max(u.NC - 1, 0) >> a.p_shift;
    const int pmask = (1 << a.p_shift) - 1;

    struct TileRegs {
        u32x4_t k[2][KL];
        u32x4_t v[VCH];
    };

    for (int win = u.ulo; win < u.uhi; win += kPidWindow) {
        const int span = min(u.uhi - win, kPidWindow);
        __syncthreads();  // the previous window is done with the page-id table
        {
            // entry 2j + h: slab (page * Hkv + kv head) of half h (16 tokens) of tile win + j
            const int n = 2 * span;
            for (int j0 = 0; j0 < n; j0 += 8 * nthreads) {
                int v[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int j = j0 + e * nthreads + tid;
                    const int tok = (win + (j >> 1)) * T + 16 * (j & 1);
                    v[e] = j < n ? pt_row[min(tok >> a.p_shift, last_page)] : 0;
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int j = j0 + e * nthreads + tid;
                    if (j < n) pid_tab[j] = checked_page(a, v[e]) * a.Hkv + u.hk;
                }
            }
        }
        __syncthreads();
        if (win == u.ulo) trace_point(a, kTrPages);
        const int nk = span > tg ? (span - tg + WT - 1) / WT : 0;
        if (nk == 0) continue;

        auto issue = [&](TileRegs& t, int k) {
            const int kc = min(k, nk - 1);
            const int j = 2 * (tg + kc * WT);
            const int slab0 = __builtin_amdgcn_readfirstlane(pid_tab[j]);
            const int slab1 = __builtin_amdgcn_readfirstlane(pid_tab[j + 1]);
            const int t0 = (win + tg + kc * WT) * T;
            const size_t base0 = ((size_t)slab0 << (a.p_shift + kLog2<D>)) + (size_t)((t0 & pmask) * D);
            const size_t base1 = ((size_t)slab1 << (a.p_shift + kLog2<D>)) + (size_t)(((t0 + 16) & pmask) * D);
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int kl = 0; kl < KL; ++kl)
                    t.k[mb][kl] = ldkv16<FP8>(a.kc, (mb ? base1 : base0) + (size_t)r16 * D + kelem<FP8>(FP8 ? 2 * kl : kl, quad));
#pragma unroll
            for (int c = 0; c < VCH; ++c) {
                const int row = c * RPC + (lane * VE) / D;  // tile row of this lane's 16 bytes
                const int col = (lane * VE) % D;
                const bool h1 = c * RPC >= 16;
                t.v[c] = ldkv16<FP8>(a.vc, (h1 ? base1 : base0) + (size_t)(row - (h1 ? 16 : 0)) * D + col);
            }
        };

        auto consume = [&](TileRegs& t, int k, bool valid, bool reissue) {
            const int t0 = (win + tg + k * WT) * T;
            f32x4_t s[NBW][2];
            if (valid) {
                // V rows into the wave's LDS tile, as bf16; on the tail tile rows past the
                // cached keys become zeros
                auto put_v = [&](bool tail) {
#pragma unroll
                    for (int c = 0; c < VCH; ++c) {
                        const int row = c * RPC + (lane * VE) / D;
                        const int col = (lane * VE) % D;
                        const bool zero = tail && t0 + row >= u.NC;
                        const u32x4_t z = {0u, 0u, 0u, 0u};
                        if constexpr (FP8) {
                            const u32x4_t lo = widen8(u32x2_t{t.v[c].x, t.v[c].y});
                            const u32x4_t hi = widen8(u32x2_t{t.v[c].z, t.v[c].w});
                            *(u32x4_t*)(vlds + row * VP + col) = zero ? z : lo;
                            *(u32x4_t*)(vlds + row * VP + col + 8) = zero ? z : hi;
                        } else {
                            *(u32x4_t*)(vlds + row * VP + col) = zero ? z : t.v[c];
                        }
                    }
                };
                if (t0 + T > u.NC)
                    put_v(true);
                else
                    put_v(false);
                bf16x8_t kf[2][KK];
#pragma unroll
                for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                    for (int kl = 0; kl < KL; ++kl) {
                        if constexpr (FP8) {
                            kf[mb][2 * kl] = __builtin_bit_cast(bf16x8_t, widen8(u32x2_t{t.k[mb][kl].x, t.k[mb][kl].y}));
                            kf[mb][2 * kl + 1] = __builtin_bit_cast(bf16x8_t, widen8(u32x2_t{t.k[mb][kl].z, t.k[mb][kl].w}));
                        } else {
                            kf[mb][kl] = __builtin_bit_cast(bf16x8_t, t.k[mb][kl]);
                        }
                    }
                w.scores(kf, s);
            }
            if (reissue) issue(t, k + 2);  // the registers are free again: keep two tiles in flight
            if (valid) {
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                bf16x8_t vf[DB];
                const uint16_t* vrow = vlds + (size_t)(4 * quad + (r16 >> 2)) * VP + 4 * (r16 & 3);
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const u32x2_t lo = lds_read_tr16(vrow + db * 16);
                    const u32x2_t hi = lds_read_tr16(vrow + 16 * VP + db * 16);
                    vf[db] = __builtin_bit_cast(bf16x8_t, u32x4_t{lo.x, lo.y, hi.x, hi.y});
                }
                w.update(s, vf, t0, a.scale_log2, quad);
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            }
        };

        // Tile A's loads come first on every path into the loop head and tile B's right
        // after, so each wait below names exactly one tile. The loop runs while a third
        // tile follows the pair, so every load it issues is a real tile; the last one or
        // two tiles are consumed after it with no further loads (re-reading a clamped
        // tile would fetch it from HBM again: the loads do not keep lines in the caches).
        TileRegs ta, tb;
        issue(ta, 0);
        int k = 0;
        for (; k + 2 < nk; k += 2) {
            issue(tb, k + 1);
            consume(ta, k, true, true);
            consume(tb, k + 1, true, false);
        }
        if (k + 1 < nk) {
            issue(tb, k + 1);
            consume(ta, k, true, false);
            consume(tb, k + 1, true, false);
        } else {
            consume(ta, k, true, false);
        }
    }
    if (a.k_block != nullptr && u.s == u.S - 1) {
        // The block keys C .. N - 1 (K <= 16 of them) from the dense arrays, as one more
        // tile at token C, consumed by token group 0; then the optional append.
        if (tg == 0) {
            w.hi_cap = u.N;
            const size_t rstride = (size_t)a.Hkv * D;
            const uint16_t* kb = a.k_block + ((size_t)u.b * a.K * a.Hkv + u.hk) * D;
            const uint16_t* vb = a.v_block + ((size_t)u.b * a.K * a.Hkv + u.hk) * D;
            bf16x8_t kf[2][KK];
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) {
                    const int i = mb * 16 + r16;
                    kf[mb][kk] = __builtin_bit_cast(bf16x8_t, i < a.K ? ldg16(kb + i * rstride + kelem<FP8>(kk, quad))
                                                                     : u32x4_t{0u, 0u, 0u, 0u});
                }
#pragma unroll
            for (int c = 0; c < D / 16; ++c) {  // 8 bf16 elements per lane
                const int row = c * (512 / D) + (lane * 8) / D;
                const int col = (lane * 8) % D;
                *(u32x4_t*)(vlds + row * VP + col) = row < a.K ? ldg16(vb + row * rstride + col) : u32x4_t{0u, 0u, 0u, 0u};
            }
            f32x4_t s[NBW][2];
            w.scores(kf, s);
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            bf16x8_t vf[DB];
            const uint16_t* vrow = vlds + (size_t)(4 * quad + (r16 >> 2)) * VP + 4 * (r16 & 3);
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const u32x2_t lo = lds_read_tr16(vrow + db * 16);
                const u32x2_t hi = lds_read_tr16(vrow + 16 * VP + db * 16);
                vf[db] = __builtin_bit_cast(bf16x8_t, u32x4_t{lo.x, lo.y, hi.x, hi.y});
            }
            w.template update<true>(s, vf, u.C, a.block_scale_log2, quad, a.block_p_mul);
        }
        if (a.append && u.rg == 0) append_block<D, FP8>(a, u);
    }
    if (wave == 0) trace_point(a, kTrLoop);
    finish_unit(a, u, w, tg, wr, WT, WR, reinterpret_cast<float*>(lds));
}

// ---------------------------------------------------------------------------------
// Shared-tile main loop for many query rows (R > 32): WR row-waves, each owning up
// to NBW row blocks, all consume every tile of the unit. Where each row-wave loading
// its own copy of a tile would leave only about one tile of unique bytes in flight
// per workgroup, here the workgroup loads each tile once: each wave moves up to LPT
// 1-KiB blocks of K and V (16 bytes per lane), DR tiles ahead of the one being
// consumed, into a three-slot LDS ring (row-major, padded pitch). One workgroup
// barrier per tile orders the ring; it waits on LDS traffic only, so the DR tiles
// of global loads stay in flight across it.
// With TG token groups the workgroup holds TG such row-wave sets, each with its own
// ring, taking every TG-th tile of the unit (group g: tiles g, g + TG, ...), so each
// wave can own two row blocks (half the LDS reads per row of a one-block wave) while
// two waves still share each SIMD. The groups' softmax states meet in LDS at the end.
// Pipelined across tiles: while a wave runs the softmax and PV product of tile t, the
// score MFMAs of tile t + 1 are already issued (its keys sit in the next ring slot), so
// the matrix cores and the vector ALUs of a SIMD work on different tiles at once.
// Every load sits at a fixed place, so each wait names exactly one tile. Loads that
// would fall past the unit's last tile, or past the tile's last block, go through a
// buffer resource with no records: the instruction runs (the wait counts stay exact)
// but reads nothing from memory and returns zeros.
template <int D, int NBW, bool WINDOWED, bool ALL_ON, int WR, int DR, bool FP8, int TG>
__global__ __launch_bounds__(64 * WR * TG, (D == 64 || NBW == 1 || TG > 1) ? 2 : 1) void shared_kernel(const KernelArgs a) {
    constexpr int NT = 64 * WR * TG;
    constexpr int EB = FP8 ? 1 : 2;       // bytes per cached element
    constexpr int LE = 16 / EB;           // elements per 16-byte lane load
    constexpr int PL = D / LE;            // lanes per tile row
    constexpr int NBLK = 2 * T * D / (64 * LE);  // 1-KiB blocks per tile: K and V, 32 rows each
    constexpr int BP = NBLK / 4;          // blocks per 16-row half of K or V
    constexpr int RPB = 64 * LE / D;      // tile rows per block
    constexpr int LPT = (NBLK + WR - 1) / WR;
    // Four row-waves: wave w moves the BP blocks of part w (one 16-row half of K or V,
    // contiguous in its page), through one buffer resource per tile.
    constexpr bool PPW = WR * BP == NBLK;
    constexpr int KP = kKPitch<D>;        // padded row pitch (bf16) of the K tile in LDS
    constexpr int VP = kVPitch<D>;        // and of the V tile
    constexpr int SLOT = T * (KP + VP);   // bf16 elements per ring slot: K tile, then V tile
    constexpr int NSLOT = 3;              // ring slots
    constexpr int DB = D / 16, KK = D / 32;
    static_assert(DR >= 2, "the prologue stages two tiles");

    extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tg = wave / WR, wr = wave - tg * WR;  // token group, row-wave inside it
    const int r16 = lane & 15, quad = lane >> 4;
    trace_point(a, kTrEntry);
    const Unit u = decode_unit<WINDOWED>(a);
    trace_point(a, kTrLength);
    WaveRows<D, NBW, WINDOWED, ALL_ON> w;
    w.init(a, u, wr * NBW, lane);
    uint16_t* ring = lds + tg * NSLOT * SLOT;  // this token group's ring
    int* pid_tab = reinterpret_cast<int*>(lds + TG * NSLOT * SLOT);

    const int32_t* pt_row = a.page_table + (size_t)u.b * a.stride;
    const int last_page = max(u.NC - 1, 0) >> a.p_shift;
    const int pmask = (1 << a.p_shift) - 1;
    // This lane's piece inside any block: row lrow of the block, columns lcol..lcol+LE-1.
    const int lrow = lane / PL, lcol = (lane % PL) * LE;
    const uint32_t lane_goff = (uint32_t)(lrow * D + lcol) * EB;  // bytes, in the cache
    const uint32_t lane_koff = (uint32_t)(lrow * KP + lcol) * 2;  // bytes, in the K tile
    const uint32_t lane_voff = (uint32_t)(lrow * VP + lcol) * 2;  // bytes, in the V tile
    const void* pool_w = (wr >> 1) ? a.vc : a.kc;                 // the pool of this wave's part (one part per wave)

    struct Stage {
        u32x4_t c[LPT];
    };

    // Key fragments (A operand of S^T = K Q^T) of the tile in ring slot `slot`.
    auto read_k = [&](int slot, bf16x8_t (&kf)[2][KK]) {
        const uint16_t* kl = ring + slot * SLOT;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int kk = 0; kk < KK; ++kk)
                kf[mb][kk] =
                    __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(kl + (mb * 16 + r16) * KP + kk * 32 + quad * 8));
    };
    // Value fragments (V^T, transposed from the row-major tile) of the tile in ring slot `slot`.
    auto read_v = [&](int slot, bf16x8_t (&vf)[DB]) {
        const uint16_t* vrow = ring + slot * SLOT + T * KP + (4 * quad + (r16 >> 2)) * VP + 4 * (r16 & 3);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const u32x2_t lo = lds_read_tr16(vrow + db * 16);
            const u32x2_t hi = lds_read_tr16(vrow + 16 * VP + db * 16);
            vf[db] = __builtin_bit_cast(bf16x8_t, u32x4_t{lo.x, lo.y, hi.x, hi.y});
        }
    };

    for (int win = u.ulo; win < u.uhi; win += kPidWindow) {
        const int span = min(u.uhi - win, kPidWindow);
        __syncthreads();  // the previous window is done with the page-id table and the ring
        {
            // entry 2j + h: slab (page * Hkv + kv head) of half h (16 tokens) of tile win + j
            const int n = 2 * span;
            for (int j0 = 0; j0 < n; j0 += 8 * NT) {
                int v[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int j = j0 + e * NT + tid;
                    const int tok = (win + (j >> 1)) * T + 16 * (j & 1);
                    v[e] = j < n ? pt_row[min(tok >> a.p_shift, last_page)] : 0;
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int j = j0 + e * NT + tid;
                    if (j < n) pid_tab[j] = checked_page(a, v[e]) * a.Hkv + u.hk;
                }
            }
        }
        __syncthreads();
        if (win == u.ulo) trace_point(a, kTrPages);
        // This group's tiles of the window: local tile t is window tile TG * t + tg. Every
        // group runs the same number of steps (the barriers are shared); a group with one
        // tile fewer idles through its last step.
        const int nk = (span - tg + TG - 1) / TG;
        const int steps = (span + TG - 1) / TG;

        // A tile is NBLK blocks of 64 16-byte pieces in four parts (K rows 0-15,
        // K rows 16-31, V rows 0-15, V rows 16-31) of BP blocks each. Row-wave w moves
        // blocks w, w + WR, ..., so each block's part, page and bases are wave-uniform
        // scalars and a lane's offset inside a block is fixed (with four row-waves, wave w
        // moves the BP blocks of part w instead). A wave's slot past the last block, and
        // every block of a tile past the unit's end, reads through an empty buffer
        // resource (zeros, no memory traffic) and is not stored; every resource ends at
        // the unit's last cached row, so rows past it load as zeros too.
        auto issue = [&](Stage& st, int t) {
            const bool real = t < nk;
            const int tc = real ? TG * t + tg : 0;  // window tile (any valid one when not real)
            if constexpr (PPW) {
                const int h = wr & 1;  // the part's 16-token half of the tile
                const int sl = __builtin_amdgcn_readfirstlane(pid_tab[2 * tc + h]);
                const int t0 = (win + tc) * T + 16 * h;
                const size_t slab = ((size_t)sl << (a.p_shift + kLog2<D>)) + (size_t)((t0 & pmask) * D);
                // The resource ends at the last cached row: rows past it read as zeros (a
                // V row there must not be a stale NaN; a K row there is masked anyway).
                // rows left from the part's first one; past 16 the part is whole (this also keeps
                // the byte count far from overflow at any allowed length)
                const int left = u.NC - t0;
                const int bytes = !real ? 0 : (left >= 16 ? BP * 64 * 16 : max(0, left) * D * EB);
                const uint64_t addr = reinterpret_cast<uint64_t>(pool_w) + slab * EB;
                const char* base = reinterpret_cast<const char*>(
                    ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(addr >> 32)) << 32) |
                    (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)addr));
                // (scalar operands: a resource built from vector registers needs a per-lane loop)
                const __amdgpu_buffer_rsrc_t rs = make_rsrc(base, __builtin_amdgcn_readfirstlane(bytes));
#pragma unroll
                for (int k = 0; k < LPT; ++k)
                    st.c[k] = __builtin_amdgcn_raw_buffer_load_b128(rs, lane_goff + k * 64 * 16, 0, kCachePolicyStream);
                return;
            }
            const int sl0 = __builtin_amdgcn_readfirstlane(pid_tab[2 * tc]);
            const int sl1 = __builtin_amdgcn_readfirstlane(pid_tab[2 * tc + 1]);
            const int t0 = (win + tc) * T;
            const size_t slab0 = ((size_t)sl0 << (a.p_shift + kLog2<D>)) + (size_t)((t0 & pmask) * D);
            const size_t slab1 = ((size_t)sl1 << (a.p_shift + kLog2<D>)) + (size_t)(((t0 + 16) & pmask) * D);
#pragma unroll
            for (int k = 0; k < LPT; ++k) {
                const int bw = wr + k * WR;
                const int b = min(bw, NBLK - 1);
                const int part = b / BP;
                const int row0 = (part & 1) * 16 + (b % BP) * RPB;  // first tile row of the block
                const char* base = static_cast<const char*>((part >> 1) ? a.vc : a.kc) +
                                   (((part & 1) ? slab1 : slab0) + (size_t)(b % BP) * RPB * D) * EB;
                // the resource ends at the last cached row: rows past it read as zeros (past
                // RPB rows the block is whole)
                const int left = u.NC - (t0 + row0);
                const int bytes = !(real && bw < NBLK) ? 0 : (left >= RPB ? 64 * 16 : max(0, left) * D * EB);
                st.c[k] = __builtin_amdgcn_raw_buffer_load_b128(make_rsrc(base, bytes), lane_goff, 0, kCachePolicyStream);
            }
        };
        auto store = [&](Stage& st, int slot) {
            char* dst = reinterpret_cast<char*>(ring + slot * SLOT);
            if constexpr (PPW) {
                // rows past the cached keys were loaded as zeros (the resource ends there)
                const int row_h = (wr & 1) * 16;  // first tile row of the wave's part
                if (wr >> 1) {
                    char* vd = dst + (T * KP + row_h * VP) * 2 + lane_voff;
#pragma unroll
                    for (int k = 0; k < LPT; ++k) {
                        if constexpr (FP8) {
                            *(u32x4_t*)(vd + k * RPB * VP * 2) = widen8(u32x2_t{st.c[k].x, st.c[k].y});
                            *(u32x4_t*)(vd + k * RPB * VP * 2 + 16) = widen8(u32x2_t{st.c[k].z, st.c[k].w});
                        } else {
                            *(u32x4_t*)(vd + k * RPB * VP * 2) = st.c[k];
                        }
                    }
                } else {
                    char* kd = dst + row_h * KP * 2 + lane_koff;
#pragma unroll
                    for (int k = 0; k < LPT; ++k) {
                        if constexpr (FP8) {
                            *(u32x4_t*)(kd + k * RPB * KP * 2) = widen8(u32x2_t{st.c[k].x, st.c[k].y});
                            *(u32x4_t*)(kd + k * RPB * KP * 2 + 16) = widen8(u32x2_t{st.c[k].z, st.c[k].w});
                        } else {
                            *(u32x4_t*)(kd + k * RPB * KP * 2) = st.c[k];
                        }
                    }
                }
                return;
            }
#pragma unroll
            for (int k = 0; k < LPT; ++k) {
                const int bw = wr + k * WR;
                if (k * WR >= NBLK - (WR - 1) && bw >= NBLK) continue;  // this wave has no block here
                const int b = bw;
                const int part = b / BP;
                const int row0 = (part & 1) * 16 + (b % BP) * RPB;  // first tile row of the block
                // rows past the cached keys were loaded as zeros (the block's resource ends there)
                char* d = dst + ((part >> 1) ? (T * KP + row0 * VP) * 2 + lane_voff : row0 * KP * 2 + lane_koff);
                if constexpr (FP8) {
                    *(u32x4_t*)d = widen8(u32x2_t{st.c[k].x, st.c[k].y});
                    *(u32x4_t*)(d + 16) = widen8(u32x2_t{st.c[k].z, st.c[k].w});
                } else {
                    *(u32x4_t*)d = st.c[k];
                }
            }
        };

        // Tile t waits in st[t % DR] until it is written to ring slot t % 3, two
        // iterations before it is consumed. The scheduling barriers keep the loads of
        // successive tiles in tile order, so the counter wait before each store covers
        // exactly the oldest tile.
        Stage st[DR];
#pragma unroll
        for (int j = 0; j < DR; ++j) {
            issue(st[j], j);
            __builtin_amdgcn_sched_barrier(0);
        }
        store(st[0], 0);
        issue(st[0], DR);
        __builtin_amdgcn_sched_barrier(0);
        store(st[1], 1);
        issue(st[1], DR + 1);
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
        // Scores of tiles t and t + 1 in two buffers that swap roles every tile (no copy
        // when DR is even; an odd DR copies the next into the current).
        f32x4_t sbuf[2][NBW][2];
        {
            bf16x8_t kf[2][KK];
            read_k(0, kf);
            w.scores(kf, sbuf[0]);
        }
        int slot = 0;  // ring slot of tile t
        for (int tb = 0; tb < steps; tb += DR) {
#pragma unroll
            for (int j = 0; j < DR; ++j) {
                const int t = tb + j;
                const int slot1 = slot == NSLOT - 1 ? 0 : slot + 1;    // tile t + 1
                const int slot2 = slot1 == NSLOT - 1 ? 0 : slot1 + 1;  // tile t + 2 (held tile t - 1)
                constexpr bool kSwap = DR % 2 == 0;
                f32x4_t(&s_cur)[NBW][2] = sbuf[kSwap ? (j & 1) : 0];
                f32x4_t(&s_next)[NBW][2] = sbuf[kSwap ? ((j + 1) & 1) : 1];
                // A wave whose one row block holds no live rows only loads (the fourth wave
                // at three row blocks).
                if (t < nk && (ALL_ON || NBW > 1 || w.on[0])) {
                    // the keys of tile t + 1 from LDS first (their latency runs under the
                    // exponent arguments of tile t), then in one straight run the scores of
                    // tile t + 1 (past the end: zeros, unused) and the probabilities and PV
                    // product of tile t (a block with no live rows computes too: no branch)
                    bf16x8_t kf[2][KK];
                    read_k(slot1, kf);
                    float y[NBW][8];
                    w.template prep<true>(s_cur, (win + TG * t + tg) * T, a.scale_log2, quad, y);
                    bf16x8_t vf[DB];
                    read_v(slot, vf);
                    w.template scores<true>(kf, s_next);
                    w.template apply<false, true>(y, vf);
                    if constexpr (!kSwap) {
#pragma unroll
                        for (int n = 0; n < NBW; ++n) {
                            s_cur[n][0] = s_next[n][0];
                            s_cur[n][1] = s_next[n][1];
                        }
                    }
                }
                store(st[(j + 2) % DR], slot2);
                issue(st[(j + 2) % DR], t + 2 + DR);
                __builtin_amdgcn_sched_barrier(0);
                __syncthreads();
                slot = slot1;
            }
        }
    }
    if (a.k_block != nullptr && u.s == u.S - 1) {
        // The block keys C .. N - 1 (K <= 16 of them) from the dense arrays into ring
        // slot 0 of token group 0 (rows past K zero), consumed as one more tile at token
        // C by that group's row-waves; then the optional append.
        __syncthreads();  // every wave is done with the ring
        const size_t rstride = (size_t)a.Hkv * D;
        const size_t b0 = ((size_t)u.b * a.K * a.Hkv + u.hk) * D;
        for (int idx = tid; idx < 2 * T * (D / 8); idx += NT) {
            const bool isv = idx >= T * (D / 8);
            const int e = isv ? idx - T * (D / 8) : idx;
            const int row = e / (D / 8), col = (e - (e / (D / 8)) * (D / 8)) * 8;
            const uint16_t* src = (isv ? a.v_block : a.k_block) + b0 + row * rstride + col;
            *(u32x4_t*)(lds + (isv ? T * KP + row * VP : row * KP) + col) =
                row < a.K ? ldg16(src) : u32x4_t{0u, 0u, 0u, 0u};
        }
        __syncthreads();
        w.hi_cap = u.N;
        if (tg == 0) {
            bf16x8_t kf[2][KK];
            read_k(0, kf);
            f32x4_t sb[NBW][2];
            w.scores(kf, sb);
            bf16x8_t vf[DB];
            read_v(0, vf);
            w.template update<true>(sb, vf, u.C, a.block_scale_log2, quad, a.block_p_mul);
        }
        if (a.append && u.rg == 0) append_block<D, FP8>(a, u);
    }
    if (wave == 0) trace_point(a, kTrLoop);
    finish_unit(a, u, w, tg, wr, TG, WR, reinterpret_cast<float*>(lds));
}

// ---------------------------------------------------------------------------------
// LSE combine of the splits. A row's D / 4 threads (4 floats each) form one split
// stream; SL streams per row (a power of two, chosen from the largest split count so
// that a thread folds at most about four splits) and 256 / (D / 4 * SL) rows per
// workgroup. With one stream a row's threads finish it from registers; with several,
// the streams' states meet in LDS behind one barrier.
template <int D>
__global__ __launch_bounds__(256) void combine_kernel(const KernelArgs a, int SL, int rows) {
    constexpr int DL = D / 4;        // threads per split stream, 4 floats each
    constexpr int NS = 256 / DL;     // split streams per workgroup (SL per row)
    __shared__ float red_acc[NS][D];
    __shared__ float red_l[NS];
    __shared__ float red_m[NS];

    const int tid = threadIdx.x;
    const int st = tid / DL, d4 = tid - st * DL;  // stream slot in the workgroup, column group
    const int rl = st / SL, sl = st - rl * SL;      // row in the workgroup, stream of the row
    const int row = blockIdx.x * (NS / SL) + rl;
    // row = (request, kv head, row rk of its R_all rows); rk lives in row group rk / R.
    int u0 = 0, S = 0, r = 0;
    size_t orow = 0;
    if (row < rows) {
        const int head = row / a.R_all, rk = row - (row / a.R_all) * a.R_all;
        const int b = head / a.Hkv, hk = head - (head / a.Hkv) * a.Hkv;
        const int rg = rk / a.R;
        r = rk - rg * a.R;
        const int pair = head * a.row_groups + rg;  // the units of that row group
        if (a.uniform_splits > 0) {  // units are laid out pair by pair: no table load
            S = a.uniform_splits;
            u0 = pair * S;
        } else {
            u0 = a.pair_table[2 * pair];
            S = a.pair_table[2 * pair + 1];
        }
        const int i = rk / a.g, l = rk - (rk / a.g) * a.g, h = hk * a.g + l;
        orow = (size_t)(b * a.K + i) * a.Hq + h;
    }
    const bool active = S > 1;  // a single split wrote its output itself

    // Each thread folds its stream's splits into a running (m, l, acc) state, so every
    // load is independent of the others. A state with m = -inf (no keys) weighs 0, and
    // 0 * NaN still carries a NaN sum through.
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    float m = kNegInf, lsum = 0.f;
    if (active) {
#pragma unroll 4
        for (int s = sl; s < S; s += SL) {
            const size_t pr = (size_t)(u0 + s) * a.R + r;
            const float ms = a.part_m[pr];
            const float ls = a.part_l[pr];
            const f32x4_t as = *(const f32x4_t*)(a.part_acc + pr * D + 4 * d4);
            const float mn = fmaxf(m, ms);
            const float wa = m == kNegInf ? 0.f : fast_exp2(m - mn);
            const float wb = ms == kNegInf ? 0.f : fast_exp2(ms - mn);
            acc = acc * wa + as * wb;
            lsum = lsum * wa + ls * wb;
            m = mn;
        }
    }
    float M = m, L, wk;
    f32x4_t o;
    if (SL == 1) {
        wk = m == kNegInf ? 0.f : fast_exp2(m - M);
        L = wk * lsum;
        o = acc * wk;
    } else {
        *(f32x4_t*)&red_acc[st][4 * d4] = acc;
        if (d4 == 0) {
            red_l[st] = lsum;
            red_m[st] = m;
        }
        __syncthreads();
        if (sl != 0) return;
        const int s0 = rl * SL;
        M = kNegInf;
        for (int k = 0; k < SL; ++k) M = fmaxf(M, red_m[s0 + k]);
        L = 0.f;
        o = f32x4_t{0.f, 0.f, 0.f, 0.f};
        for (int k = 0; k < SL; ++k) {
            wk = red_m[s0 + k] == kNegInf ? 0.f : fast_exp2(red_m[s0 + k] - M);
            L += wk * red_l[s0 + k];
            o += *(const f32x4_t*)&red_acc[s0 + k][4 * d4] * wk;
        }
    }
    if (!active) return;
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = L == 0.f ? 0.f : o[j] / L;  // no keys: zeros; a NaN sum stays NaN
    const uint32_t lo = f32_to_bf16_rne(v[0]) | ((uint32_t)f32_to_bf16_rne(v[1]) << 16);
    const uint32_t hi = f32_to_bf16_rne(v[2]) | ((uint32_t)f32_to_bf16_rne(v[3]) << 16);
    *(u32x2_t*)(a.out + orow * D + 4 * d4) = u32x2_t{lo, hi};
    if (d4 == 0 && a.lse) a.lse[orow] = L == 0.f ? kNegInf : M + log2f(L);
}

// Dynamic LDS above 64 KiB needs the kernel's limit raised, once per device (the
// attribute applies to the current device). Devices past the table are raised on
// every launch.
constexpr int kLdsGrantDevices = 64;
struct LdsGrant {
    std::atomic<size_t> bytes[kLdsGrantDevices];  // static storage: starts at zero
};

// G-way log-sum-exp merge of normalised results of the same rows over disjoint key
// sets (the combine a context-parallel split runs after gathering every shard's out
// and base-2 LSE): M = max lse_g, w_g = 2^(lse_g - M), out = sum w_g out_g / sum w_g,
// lse = M + log2 sum w_g. A part with no keys (lse = -inf) weighs 0; a NaN part makes
// the row NaN. Each thread owns 8 elements (16 bytes) of one row.
template <int D>
__global__ __launch_bounds__(256) void merge_kernel(int parts, int64_t rows, const uint16_t* part_out,
                                                   const float* part_lse, uint16_t* out, float* lse) {
    constexpr int TPR = D / 8;      // threads per row
    constexpr int RPB = 256 / TPR;  // rows per workgroup
    const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
    const int c = (threadIdx.x % TPR) * 8;
    if (row >= rows) return;
    float M = kNegInf;
    for (int g = 0; g < parts; ++g) M = fmaxf(M, part_lse[(int64_t)g * rows + row]);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float L = 0.f;
    for (int g = 0; g < parts; ++g) {
        const float lg = part_lse[(int64_t)g * rows + row];
        const float w = lg == kNegInf ? 0.f : fast_exp2(lg - M);
        const u32x4_t v = ldg16(part_out + ((int64_t)g * rows + row) * D + c);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            acc[2 * k] += w * __uint_as_float(v[k] << 16);
            acc[2 * k + 1] += w * __uint_as_float(v[k] & 0xFFFF0000u);
        }
        L += w;
    }
    const float inv = L == 0.f ? 0.f : 1.f / L;  // no keys in any part: zeros; a NaN sum stays NaN
    u32x4_t o;
#pragma unroll
    for (int k = 0; k < 4; ++k)
        o[k] = f32_to_bf16_rne(acc[2 * k] * inv) | ((uint32_t)f32_to_bf16_rne(acc[2 * k + 1] * inv) << 16);
    *(u32x4_t*)(out + row * D + c) = o;
    if (c == 0 && lse) lse[row] = L == 0.f ? kNegInf : M + log2f(L);
}

template <typename F>
hipError_t launch_with_lds(F fn, int units, int threads, size_t lds, const KernelArgs& args, hipStream_t stream,
                           LdsGrant& grant) {
    if (lds > 65536) {
        int dev = -1;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return e;
        const bool tracked = dev >= 0 && dev < kLdsGrantDevices;
        if (!tracked || grant.bytes[dev].load(std::memory_order_relaxed) < lds) {
            e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            if (e != hipSuccess) return e;
            if (tracked) {
                size_t cur = grant.bytes[dev].load(std::memory_order_relaxed);
                while (cur < lds && !grant.bytes[dev].compare_exchange_weak(cur, lds, std::memory_order_relaxed)) {
                }
            }
        }
    }
    hipLaunchKernelGGL(fn, dim3(units), dim3(threads), lds, stream, args);
    return hipGetLastError();
}

template <int D, int NBW, bool W, bool ALL_ON, bool FP8>
hipError_t launch_stream(const KernelShape& s, int units, const KernelArgs& args, hipStream_t stream) {
    static LdsGrant grant;
    constexpr int MAXT = D == 64 ? 512 : 256;  // D = 128 keeps workgroups small so a wave may use 512 registers
    return launch_with_lds(stream_kernel<D, NBW, W, ALL_ON, MAXT, FP8>, units, 64 * s.row_waves * s.token_groups,
                           s.lds_bytes, args, stream, grant);
}

// Tiles in flight per lane: about 96 registers of staged loads for a wave alone on
// its SIMD (D = 128, two row blocks), 64 where two waves share a SIMD, at most 8.
// Two row blocks with two waves per SIMD (token groups) leave room for two.
constexpr int shared_depth(int D, int NBW, int WR, bool FP8, int TG) {
    const int lpt = ((FP8 ? D / 16 : D / 8) + WR - 1) / WR;  // 1-KiB blocks per wave per tile
    const int dr = (D == 128 && NBW == 2 && TG > 1) ? 2 : ((D == 128 && NBW == 2) ? 24 : 16) / lpt;
    return dr < 2 ? 2 : (dr > 8 ? 8 : dr);
}

template <int D, int NBW, int WR, bool W, bool ALL_ON, bool FP8, int TG>
hipError_t launch_shared(const KernelShape& s, int units, const KernelArgs& args, hipStream_t stream) {
    static LdsGrant grant;
    return launch_with_lds(shared_kernel<D, NBW, W, ALL_ON, WR, shared_depth(D, NBW, WR, FP8, TG), FP8, TG>, units,
                           64 * WR * TG, s.lds_bytes, args, stream, grant);
}

template <bool W, bool FP8>
hipError_t dispatch(const KernelShape& s, int units, const KernelArgs& args, hipStream_t stream) {
    if (s.shared) {
#define BA_SHARED(D_, NBW_, WR_, TG_)                                                                   \
    if (s.head_dim == D_ && s.nbw == NBW_ && s.row_waves == WR_ && s.token_groups == TG_)               \
        return s.all_on ? launch_shared<D_, NBW_, WR_, W, true, FP8, TG_>(s, units, args, stream)       \
                        : launch_shared<D_, NBW_, WR_, W, false, FP8, TG_>(s, units, args, stream);
#define BA_SHARED1(D_, WR_)                                                                             \
    if (s.head_dim == D_ && s.nbw == 1 && s.row_waves == WR_ && s.token_groups == 1)                    \
        return launch_shared<D_, 1, WR_, W, true, FP8, 1>(s, units, args, stream);
        BA_SHARED(64, 2, 2, 1)
        BA_SHARED(64, 2, 3, 1)
        BA_SHARED(64, 2, 4, 1)
        BA_SHARED(128, 2, 2, 1)
        BA_SHARED(128, 2, 3, 1)
        BA_SHARED(128, 2, 4, 1)
        BA_SHARED(128, 2, 4, 2)
        BA_SHARED1(128, 3)
        BA_SHARED(128, 1, 4, 1)
        BA_SHARED(128, 1, 4, 2)
        BA_SHARED1(128, 5)
        BA_SHARED1(128, 6)
        BA_SHARED1(128, 7)
        BA_SHARED1(128, 8)
#undef BA_SHARED
#undef BA_SHARED1
        return hipErrorInvalidValue;
    }
#define BA_CASE(D_, NBW_)                                                                               \
    if (s.head_dim == D_ && s.nbw == NBW_)                                                              \
        return s.all_on ? launch_stream<D_, NBW_, W, true, FP8>(s, units, args, stream)                 \
                        : launch_stream<D_, NBW_, W, false, FP8>(s, units, args, stream);
    BA_CASE(64, 1)
    BA_CASE(64, 2)
    BA_CASE(128, 1)
    BA_CASE(128, 2)
#undef BA_CASE
    return hipErrorInvalidValue;
}

}  // namespace
}  // namespace blockattn
