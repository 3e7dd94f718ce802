// gfx950 kernels for draft-block paged attention.
//
// partial_kernel (split-KV partial attention). One workgroup = one work unit:
//   a range of 32-token key tiles of one (request b, kv head). Its waves form
//   WT "token groups" that stream different tiles, and each token group has WR
//   "row waves" that share one tile through LDS and own NBW 16-row blocks of the
//   R = K * group query rows each. Per tile:
//     - the K and V slabs (32 rows x D, contiguous inside an HND page) come in as
//       coalesced 16-byte global loads, one tile ahead in registers, and are
//       written to a double-buffered LDS tile (K row-major, V transposed so the
//       tokens become the MFMA reduction dimension);
//     - S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (tokens are the M dimension, the
//       query rows the N dimension, so each lane owns one query row of S^T and
//       the softmax statistics stay in-lane);
//     - online softmax in exp2 space (scores pre-multiplied by sm_scale*log2 e),
//       masks only on edge tiles; V rows past the sequence end are zeroed by
//       select, so stale cache slots (even NaN) cannot leak through 0 * NaN;
//     - O^T += V^T P^T on the same MFMA with P rounded to bf16; the P operand is
//       exactly the lane's own S^T accumulator registers (no shuffles).
//   At the end the token groups merge through LDS and the unit writes fp32
//   partial (acc, m, l). This is the split-KV ("flash-decoding") partial step
//   of TensorRT-LLM PR #16150 (paged DFlash cross-attention, commit "rework
//   flash-decoding style") and the multi-CTA split-KV of PR #20374, redone
//   for 64-wide wavefronts, MFMA tiles and HND pages.
//
// combine_kernel (LSE combine over the splits, plus the fused future-block-key
//   merge of the windowed form). One workgroup per output row (b, i, h).
//   M = max_s m_s, w_s = 2^(m_s - M), out = sum w_s acc_s / sum w_s l_s,
//   lse2 = M + log2(sum w_s l_s). For the windowed form it then scores the block
//   keys after the query (at most K - 1, read from the paged cache), forms their
//   (out_f, lse_f) and merges: lse = lse_c (+) lse_f, out = out_c + w (out_f -
//   out_c) with w = 2^(lse_f - lse), the sigmoid/lerp form of PR #21130's merge
//   formulation table. It writes bf16 out (round to nearest even) and fp32 lse.
#include "internal.h"

#include <math.h>

namespace blockattn {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

template <int D, int NBW, int CPW, bool WINDOWED>
__global__ __launch_bounds__(512) void partial_kernel(const PartialArgs a) {
    constexpr int T = kTileTokens;
    constexpr int KP = D + 8;  // padded pitch of the K tile (bf16 elements)
    constexpr int VP = T + 8;  // padded pitch of the transposed V tile
    constexpr int KT = T * KP;
    constexpr int BUF = KT + D * VP;
    constexpr int NCH = D / 8;           // 1-KiB chunks of a tile, K then V
    constexpr int HALF = NCH / 2;        // chunks per tensor
    constexpr int RPC = 1024 / (2 * D);  // tile rows per chunk
    constexpr int DB = D / 16;           // 16-wide d blocks of O^T
    constexpr int KK = D / 32;           // 32-deep k steps of S^T

    extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int WR = a.row_waves, WT = a.token_groups;
    const int tg = wave / WR;
    const int wr = wave - tg * WR;
    const int r16 = lane & 15, quad = lane >> 4;
    uint16_t* tg_lds = lds + (size_t)tg * 2 * BUF;

    const WorkItem wi = a.work[blockIdx.x];
    const int b = wi.b, hk = wi.hk;
    const int N = clampi(a.seq_lens[b], a.K, a.stride * a.P);
    const int C = N - a.K;
    const bool left_win = WINDOWED && a.window_left > 0;
    const int key_lo = left_win ? max(0, C - a.window_left + 1) : 0;
    const int tb = key_lo / T, te = (N + T - 1) / T, nt = te - tb;
    const int ulo = tb + (int)((int64_t)wi.s * nt / wi.S);
    const int uhi = tb + (int)((int64_t)(wi.s + 1) * nt / wi.S);

    // Query fragments (B operand of S^T = K Q^T) and per-row key bounds.
    bf16x8_t qf[NBW][KK];
    int row_lo[NBW], row_hi[NBW];
    bool blk_on[NBW];
#pragma unroll
    for (int n = 0; n < NBW; ++n) {
        const int nb = wr * NBW + n;
        const int r = nb * 16 + r16;
        blk_on[n] = nb * 16 < a.R;
        const bool live = r < a.R;
        const int i = live ? r / a.g : a.K - 1;
        const int l = live ? r - (r / a.g) * a.g : 0;
        const uint16_t* qrow = a.q + ((size_t)(b * a.K + i) * a.Hq + hk * a.g + l) * D;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            u32x4_t v = live ? *(const u32x4_t*)(qrow + kk * 32 + quad * 8) : u32x4_t{0u, 0u, 0u, 0u};
            qf[n][kk] = __builtin_bit_cast(bf16x8_t, v);
        }
        const int p = C + i;
        row_lo[n] = left_win ? max(0, p - a.window_left + 1) : 0;
        row_hi[n] = WINDOWED ? p : N - 1;
    }
    const int lo_max = left_win ? max(0, C + a.K - a.window_left) : 0;
    const int hi_min = WINDOWED ? C : N - 1;

    f32x4_t acc[NBW][DB];
    float m_run[NBW], l_run[NBW];
#pragma unroll
    for (int n = 0; n < NBW; ++n) {
        m_run[n] = kNegInf;
        l_run[n] = 0.f;
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[n][db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    const int32_t* pt_row = a.page_table + (size_t)b * a.stride;
    const int last_page = (N - 1) / a.P;
    const size_t head_elems = (size_t)a.P * D;
    u32x4_t pre[CPW];

    // Issue the global loads of one tile into registers. Each 16-token half of the
    // tile is contiguous inside one page; a chunk never straddles the halves.
    auto prefetch = [&](int tile) {
        const int t0 = tile * T;
        const int lp0 = min(t0 / a.P, last_page);
        const int lp1 = min((t0 + 16) / a.P, last_page);
        const int pid0 = clampi(pt_row[lp0], 0, a.num_pages - 1);
        const int pid1 = clampi(pt_row[lp1], 0, a.num_pages - 1);
        const size_t base0 = ((size_t)pid0 * a.Hkv + hk) * head_elems + (size_t)(t0 % a.P) * D;
        const size_t base1 = ((size_t)pid1 * a.Hkv + hk) * head_elems + (size_t)((t0 + 16) % a.P) * D;
#pragma unroll
        for (int ci = 0; ci < CPW; ++ci) {
            const int c = wr + ci * WR;
            if (c < NCH) {
                const bool is_v = c >= HALF;
                const int cc = is_v ? c - HALF : c;
                const int off = cc * 512 + lane * 8;  // bf16 elements inside the tensor tile
                const int row = off / D, col = off - (off / D) * D;
                const bool h1 = row >= 16;
                const size_t base = (h1 ? base1 : base0) + (size_t)(row - (h1 ? 16 : 0)) * D + col;
                pre[ci] = *(const u32x4_t*)((is_v ? a.vc : a.kc) + base);
            }
        }
    };

    // Move the prefetched registers of one tile into an LDS buffer.
    auto store = [&](int tile, uint16_t* buf) {
        const int t0 = tile * T;
#pragma unroll
        for (int ci = 0; ci < CPW; ++ci) {
            const int c = wr + ci * WR;
            if (c < NCH) {
                const int cc = c < HALF ? c : c - HALF;
                const int off = cc * 512 + lane * 8;
                const int row = off / D, col = off - (off / D) * D;
                if (c < HALF) {
                    *(u32x4_t*)(buf + row * KP + col) = pre[ci];
                } else {
                    const u32x4_t v = (t0 + row < N) ? pre[ci] : u32x4_t{0u, 0u, 0u, 0u};
                    uint16_t* vt = buf + KT + col * VP + row;
#pragma unroll
                    for (int e = 0; e < 8; ++e) vt[e * VP] = (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
                }
            }
        }
    };

    auto compute = [&](int tile, const uint16_t* buf) {
        const int t0 = tile * T;
        bf16x8_t kf[2][KK];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int kk = 0; kk < KK; ++kk)
                kf[mb][kk] = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(buf + (mb * 16 + r16) * KP + kk * 32 + quad * 8));
        bf16x8_t vf[DB];
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const uint16_t* vrow = buf + KT + (db * 16 + r16) * VP;
            const u32x2_t lo = *(const u32x2_t*)(vrow + 4 * quad);
            const u32x2_t hi = *(const u32x2_t*)(vrow + 16 + 4 * quad);
            vf[db] = __builtin_bit_cast(bf16x8_t, u32x4_t{lo.x, lo.y, hi.x, hi.y});
        }
        const bool edge = (t0 < lo_max) || (t0 + T - 1 > hi_min);
#pragma unroll
        for (int n = 0; n < NBW; ++n) {
            if (!blk_on[n]) continue;
            f32x4_t s[2];
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) {
                s[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) s[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[mb][kk], qf[n][kk], s[mb], 0, 0, 0);
            }
            float x[8];
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int j = 0; j < 4; ++j) x[mb * 4 + j] = s[mb][j] * a.scale_log2;
            if (edge) {
#pragma unroll
                for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int tok = t0 + mb * 16 + quad * 4 + j;
                        if (tok < row_lo[n] || tok > row_hi[n]) x[mb * 4 + j] = kNegInf;
                    }
            }
            float mx = x[0];
#pragma unroll
            for (int k = 1; k < 8; ++k) mx = fmaxf(mx, x[k]);
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float m_new = fmaxf(m_run[n], mx);
            const float m_use = m_new == kNegInf ? 0.f : m_new;
            const float alpha = fast_exp2(m_run[n] - m_use);
            float p[8];
            float psum = 0.f;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                p[k] = fast_exp2(x[k] - m_use);
                psum += p[k];
            }
            l_run[n] = l_run[n] * alpha + psum;
            m_run[n] = m_new;
            bf16x8_t pb;
#pragma unroll
            for (int k = 0; k < 8; ++k) pb[k] = (__bf16)p[k];
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                acc[n][db] *= alpha;
                acc[n][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[db], pb, acc[n][db], 0, 0, 0);
            }
        }
    };

    const int n_iter = uhi > ulo ? (uhi - ulo + WT - 1) / WT : 0;
    int tile = ulo + tg;
    if (n_iter > 0 && tile < uhi) prefetch(tile);
    for (int it = 0; it < n_iter; ++it) {
        uint16_t* buf = tg_lds + (it & 1) * BUF;
        const bool valid = tile < uhi;
        if (valid) store(tile, buf);
        __syncthreads();
        const int next = tile + WT;
        if (next < uhi) prefetch(next);
        if (valid) compute(tile, buf);
        tile = next;
    }

    // Row sums were kept per lane; the four lanes of a row hold disjoint tokens.
#pragma unroll
    for (int n = 0; n < NBW; ++n) {
        l_run[n] += __shfl_xor(l_run[n], 16);
        l_run[n] += __shfl_xor(l_run[n], 32);
    }

    // Merge the token groups through LDS and write this unit's partial state.
    constexpr int MP = D + 4;  // floats per row slot: acc[D], m, l, pad
    __syncthreads();
    float* mg = reinterpret_cast<float*>(lds);
#pragma unroll
    for (int n = 0; n < NBW; ++n) {
        float* slot = mg + ((size_t)((tg * WR + wr) * NBW + n) * 16 + r16) * MP;
#pragma unroll
        for (int db = 0; db < DB; ++db) *(f32x4_t*)(slot + db * 16 + quad * 4) = acc[n][db];
        if (quad == 0) {
            slot[D] = m_run[n];
            slot[D + 1] = l_run[n];
        }
    }
    __syncthreads();
    const size_t unit_row0 = (size_t)blockIdx.x * a.R;
    const int per_tg = WR * NBW * 16 * MP;
    for (int idx = threadIdx.x; idx < a.R * D; idx += blockDim.x) {
        const int r = idx / D, d = idx - (idx / D) * D;
        const int nb = r >> 4;
        const int wr_r = nb / NBW, n_r = nb - wr_r * NBW;
        const int off = ((wr_r * NBW + n_r) * 16 + (r & 15)) * MP;
        float M = kNegInf;
        for (int t = 0; t < WT; ++t) M = fmaxf(M, mg[t * per_tg + off + D]);
        float L = 0.f, A = 0.f;
        if (M != kNegInf) {
            for (int t = 0; t < WT; ++t) {
                const float w = fast_exp2(mg[t * per_tg + off + D] - M);
                L += w * mg[t * per_tg + off + D + 1];
                A += w * mg[t * per_tg + off + d];
            }
        }
        a.part_acc[(unit_row0 + r) * D + d] = A;
        if (d == 0) {
            a.part_m[unit_row0 + r] = M;
            a.part_l[unit_row0 + r] = L;
        }
    }
}

template <int D, bool MERGE>
__global__ __launch_bounds__(256) void combine_kernel(const CombineArgs a) {
    constexpr int DL = D / 4;     // threads per split row, 4 floats each
    constexpr int SL = 256 / DL;  // splits reduced in parallel
    __shared__ float red_acc[SL][D];
    __shared__ float red_l[SL];
    __shared__ float red_m[4];
    __shared__ float o_c[D];
    __shared__ float s_f[16];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int row = blockIdx.x;
    const int pair = row / a.R, r = row - (row / a.R) * a.R;
    const int b = pair / a.Hkv, hk = pair - (pair / a.Hkv) * a.Hkv;
    const int u0 = a.pair_table[2 * pair], S = a.pair_table[2 * pair + 1];
    const int i = r / a.g, l = r - (r / a.g) * a.g, h = hk * a.g + l;
    const size_t orow = (size_t)(b * a.K + i) * a.Hq + h;

    float mloc = kNegInf;
    for (int s = tid; s < S; s += 256) mloc = fmaxf(mloc, a.part_m[(size_t)(u0 + s) * a.R + r]);
    for (int o = 32; o > 0; o >>= 1) mloc = fmaxf(mloc, __shfl_xor(mloc, o));
    if (lane == 0) red_m[wave] = mloc;
    __syncthreads();
    const float M = fmaxf(fmaxf(red_m[0], red_m[1]), fmaxf(red_m[2], red_m[3]));

    const int d4 = tid % DL, sl = tid / DL;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    float lsum = 0.f;
    if (M != kNegInf) {
        for (int s = sl; s < S; s += SL) {
            const size_t pr = (size_t)(u0 + s) * a.R + r;
            const float w = fast_exp2(a.part_m[pr] - M);
            acc += w * *(const f32x4_t*)(a.part_acc + pr * D + 4 * d4);
            lsum += w * a.part_l[pr];
        }
    }
    *(f32x4_t*)&red_acc[sl][4 * d4] = acc;
    if (d4 == 0) red_l[sl] = lsum;
    __syncthreads();
    float L = 0.f;
    for (int k = 0; k < SL; ++k) L += red_l[k];
    if (tid < D) {
        float o = 0.f;
        for (int k = 0; k < SL; ++k) o += red_acc[k][tid];
        o_c[tid] = L > 0.f ? o / L : 0.f;
    }
    float lse = L > 0.f ? M + log2f(L) : kNegInf;
    __syncthreads();

    if (MERGE) {
        const int N = clampi(a.seq_lens[b], a.K, a.stride * a.P);
        const int p = N - a.K + i;
        const int f_hi = a.window_right < 0 ? N - 1 : min(N - 1, p + a.window_right);
        const int nf = f_hi - p;
        if (nf > 0) {
            const int32_t* pt_row = a.page_table + (size_t)b * a.stride;
            const uint16_t* qrow = a.q + orow * D;
            if (wave == 0) {
                for (int f = 0; f < nf; ++f) {
                    const int j = p + 1 + f;
                    const int pid = clampi(pt_row[j / a.P], 0, a.num_pages - 1);
                    const uint16_t* krow = a.kc + (((size_t)pid * a.Hkv + hk) * a.P + (j % a.P)) * D;
                    float dot = 0.f;
                    for (int d = lane; d < D; d += 64) dot += bf16_to_f32(qrow[d]) * bf16_to_f32(krow[d]);
                    for (int o = 32; o > 0; o >>= 1) dot += __shfl_xor(dot, o);
                    if (lane == 0) s_f[f] = dot * a.scale_log2;
                }
            }
            __syncthreads();
            float mf = kNegInf;
            for (int f = 0; f < nf; ++f) mf = fmaxf(mf, s_f[f]);
            float z = 0.f;
            for (int f = 0; f < nf; ++f) z += fast_exp2(s_f[f] - mf);
            const float lse_f = mf + log2f(z);
            const float hi2 = fmaxf(lse, lse_f), lo2 = fminf(lse, lse_f);
            const float merged = hi2 + log2f(1.f + fast_exp2(lo2 - hi2));
            const float wf = fast_exp2(lse_f - merged);
            if (tid < D) {
                float of = 0.f;
                for (int f = 0; f < nf; ++f) {
                    const int j = p + 1 + f;
                    const int pid = clampi(pt_row[j / a.P], 0, a.num_pages - 1);
                    const uint16_t* vrow = a.vc + (((size_t)pid * a.Hkv + hk) * a.P + (j % a.P)) * D;
                    of += fast_exp2(s_f[f] - lse_f) * bf16_to_f32(vrow[tid]);
                }
                o_c[tid] = o_c[tid] + wf * (of - o_c[tid]);
            }
            lse = merged;
            __syncthreads();
        }
    }

    if (tid < D) a.out[orow * D + tid] = f32_to_bf16_rne(o_c[tid]);
    if (tid == 0 && a.lse) a.lse[orow] = lse;
}

template <int D, int NBW, int CPW, bool W>
hipError_t launch_partial_t(const KernelShape& shape, int units, const PartialArgs& args, hipStream_t stream) {
    auto fn = partial_kernel<D, NBW, CPW, W>;
    static size_t attr_bytes = 0;  // largest dynamic LDS size granted so far
    if (shape.lds_bytes > 65536 && shape.lds_bytes > attr_bytes) {
        hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)shape.lds_bytes);
        if (e != hipSuccess) return e;
        attr_bytes = shape.lds_bytes;
    }
    const int threads = 64 * shape.row_waves * shape.token_groups;
    hipLaunchKernelGGL(fn, dim3(units), dim3(threads), shape.lds_bytes, stream, args);
    return hipGetLastError();
}

template <bool W>
hipError_t dispatch_partial(const KernelShape& s, int units, const PartialArgs& args, hipStream_t stream) {
#define BA_CASE(D_, NBW_, CPW_)                                                      \
    if (s.head_dim == D_ && s.nbw == NBW_ && s.cpw == CPW_)                          \
        return launch_partial_t<D_, NBW_, CPW_, W>(s, units, args, stream);
    BA_CASE(64, 1, 4)
    BA_CASE(64, 1, 8)
    BA_CASE(64, 2, 4)
    BA_CASE(64, 2, 8)
    BA_CASE(128, 1, 4)
    BA_CASE(128, 1, 8)
#undef BA_CASE
    return hipErrorInvalidValue;
}

}  // namespace

size_t partial_lds_bytes(int head_dim, int nbw, int row_waves, int token_groups) {
    const size_t buf = (size_t)kTileTokens * (head_dim + 8) + (size_t)head_dim * (kTileTokens + 8);
    const size_t tiles = (size_t)token_groups * 2 * buf * sizeof(uint16_t);
    const size_t merge = (size_t)token_groups * row_waves * nbw * 16 * (head_dim + 4) * sizeof(float);
    return tiles > merge ? tiles : merge;
}

hipError_t launch_partial(const KernelShape& shape, bool windowed, int units, const PartialArgs& args,
                          hipStream_t stream) {
    return windowed ? dispatch_partial<true>(shape, units, args, stream)
                    : dispatch_partial<false>(shape, units, args, stream);
}

hipError_t launch_combine(int head_dim, bool merge, int rows, const CombineArgs& args, hipStream_t stream) {
    if (head_dim == 64) {
        if (merge) hipLaunchKernelGGL((combine_kernel<64, true>), dim3(rows), dim3(256), 0, stream, args);
        else hipLaunchKernelGGL((combine_kernel<64, false>), dim3(rows), dim3(256), 0, stream, args);
    } else if (head_dim == 128) {
        if (merge) hipLaunchKernelGGL((combine_kernel<128, true>), dim3(rows), dim3(256), 0, stream, args);
        else hipLaunchKernelGGL((combine_kernel<128, false>), dim3(rows), dim3(256), 0, stream, args);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace blockattn
