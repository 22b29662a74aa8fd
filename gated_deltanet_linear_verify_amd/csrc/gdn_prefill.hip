// gdn_prefill.hip - chunked (WY / UT form) prefill of the gated delta rule on MFMA (gfx950).
//
// A prefill-only call has no per-position capture (lucebox-hub internal.h, create_target_cache
// prefill_only).  The recurrence S_t = rho_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
// (Yang, Kautz & Hatamizadeh 2024) is evaluated 64 tokens at a time.  Within a chunk with start
// state S (d_v x d_k), Gamma_t = sum_{s<=t} g_s, gamma_t = exp(Gamma_t):
//   A[t][s] = beta_t exp(Gamma_t - Gamma_s) (k_t . k_s)   for s < t      (strictly lower)
//   T       = (I + A)^-1
//   Y       = diag(beta) V - diag(beta gamma) K S^T
//   U       = T Y                       (the rows u_t of the rank-1 updates S += u_t k_t^T)
//   P[t][s] = exp(Gamma_t - Gamma_s) (q_t . k_s)          for s <= t
//   O       = diag(gamma) Q S^T + P U                     (o_t = S_t q_t)
//   S'      = gamma_C S + U^T diag(gamma_C / gamma) K
// which is the token recurrence unrolled (u_t = beta_t (v_t - rho_t S_{t-1} k_t)); only ratios
// exp(Gamma_t - Gamma_s) with s <= t and gamma_t <= 1 are ever formed.
//
// Kernel 1 (chunk scan): one workgroup per (value head, block of 16 value rows).  Rows of S are
// independent given the keys, so the blocks never communicate; each walks the chunks in order with
// its S block in LDS.  Dense products run on v_mfma_f32_16x16x32_bf16 with each fp32 operand
// split into bf16 hi + lo parts (a b ~ a_hi b_hi + a_hi b_lo + a_lo b_hi, ~2^-16 relative), so the
// fp32 state is not rounded to bf16; with fp32 activations the products run on the fp32 MFMA.  T comes from a blocked fp32 forward substitution.
// Kernel 2 (epilogue): RMS norm over d_v + SiLU(z) gate of every token (the d_v blocks of kernel 1
// meet here through an fp32 workspace), and the conv state after the last token.
#include "gdn_device.h"
#include "gdn_internal.h"

#include <type_traits>

namespace gdn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kChunk = 64;  // tokens per chunk
constexpr int kDB = 16;     // value rows per workgroup
constexpr int kPThreads = 256;

__device__ __forceinline__ f4 mfma16(bf16x8 a, bf16x8 b, f4 c)
{
#if defined(__HIP_DEVICE_COMPILE__)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
#else
    (void)a;
    (void)b;
    return c;
#endif
}

__device__ __forceinline__ f4 mfma4f32(float a, float b, f4 c)
{
#if defined(__HIP_DEVICE_COMPILE__)
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
#else
    (void)a;
    (void)b;
    return c;
#endif
}

// 8 fp32 values -> bf16 hi and lo parts (hi = RNE(x), lo = RNE(x - hi)).
__device__ __forceinline__ void split8(const float (&x)[8], bf16x8 &hi, bf16x8 &lo)
{
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const __bf16 h = (__bf16)x[j];
        hi[j] = h;
        lo[j] = (__bf16)(x[j] - (float)h);
    }
}

__device__ __forceinline__ void load8(const float *p, float (&x)[8])
{
    const f4 a = *reinterpret_cast<const f4 *>(p);
    const f4 b = *reinterpret_cast<const f4 *>(p + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        x[j] = a[j];
        x[4 + j] = b[j];
    }
}

// One 32-deep step of a 16x16 product.  Lane l holds a[e] = A[l % 16][8 (l / 16) + e] and
// b[e] = B[8 (l / 16) + e][l % 16] of the 16x32 and 32x16 operands; the result rows are
// 4 (l / 16) + r, columns l % 16.
// F32: eight v_mfma_f32_16x16x4_f32, step e taking k index 8 kk + e for the instruction's kk = l / 16
// (fp32 products, the precision of the all-fp32 path).  Otherwise one 16x16x32 bf16 MFMA per
// pair of bf16 parts: a b ~ a_lo b_hi + a_hi b_lo + a_hi b_hi (the a_lo b_lo term, ~2^-16 of a b,
// is dropped), smallest terms first.
template <bool F32>
__device__ __forceinline__ f4 mma8(const float (&a)[8], const float (&b)[8], f4 acc)
{
    if constexpr (F32) {
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = mfma4f32(a[e], b[e], acc);
    } else {
        bf16x8 ah, al, bh, bl;
        split8(a, ah, al);
        split8(b, bh, bl);
        acc = mfma16(al, bh, acc);
        acc = mfma16(ah, bl, acc);
        acc = mfma16(ah, bh, acc);
    }
    return acc;
}

// acc += A(16x32 at row r0, col k0 of a row-major [.][lda] matrix) * B, where B (32x16) is given
// transposed: Bt row-major [n][ldb], block at row n0, col k0.
template <bool F32>
__device__ __forceinline__ f4 mma_tile(const float *A, int lda, int r0, const float *Bt, int ldb, int n0, int k0,
                                       f4 acc, int lane)
{
    float av[8], bv[8];
    load8(A + (r0 + (lane & 15)) * lda + k0 + (lane >> 4) * 8, av);
    load8(Bt + (n0 + (lane & 15)) * ldb + k0 + (lane >> 4) * 8, bv);
    return mma8<F32>(av, bv, acc);
}

template <int D, typename act_t>
struct PrefillLds {
    static constexpr int C = kChunk;
    static constexpr int NCH = 2 * D + kDB;  // q | k | v-block channels
    static constexpr size_t q = 0;                                   // [C][D]
    static constexpr size_t k = q + sizeof(float) * C * D;           // [C][D]
    static constexpr size_t kt = k + sizeof(float) * C * D;          // [D][C]
    static constexpr size_t vb = kt + sizeof(float) * D * C;         // [C][DB]
    static constexpr size_t s = vb + sizeof(float) * C * kDB;        // [DB][D]   the state block
    static constexpr size_t tm = s + sizeof(float) * kDB * D;        // [C][C]    A, then T
    static constexpr size_t pm = tm + sizeof(float) * C * C;         // [C][C]    scratch, then P
    static constexpr size_t yt = pm + sizeof(float) * C * C;         // [DB][C]
    static constexpr size_t ut = yt + sizeof(float) * kDB * C;       // [DB][C]
    static constexpr size_t work_end = ut + sizeof(float) * kDB * C;
    static constexpr size_t raw_bytes = sizeof(act_t) * (C + 3) * NCH;  // staged rows, aliases tm..
    static constexpr size_t sc = (tm + raw_bytes > work_end ? tm + raw_bytes : work_end);
    static constexpr size_t total = sc + sizeof(float) * 4 * C;      // Gamma, gamma, beta, decay-to-end
};

template <int D, bool ACT_BF16, bool QKN>
__global__ __launch_bounds__(kPThreads) void prefill_chunk_kernel(PrefillArgs a)
{
    using act_t = typename std::conditional<ACT_BF16, uint16_t, float>::type;
    using L = PrefillLds<D, act_t>;
    constexpr bool F32 = !ACT_BF16;  // fp32 activations: fp32 MFMA products
    constexpr int C = kChunk;
    constexpr int NCH = L::NCH;
    constexpr int VEC = 16 / (int)sizeof(act_t);
    constexpr int NB = D / kDB;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int R = a.n_vh / a.n_kh;

    const int h = blockIdx.x / NB, blk = blockIdx.x % NB;
    const int hk = h / R;
    const int T = a.T;
    const int Cc = a.C;  // conv channels
    const int q0 = hk * D, k0 = a.n_kh * D + hk * D, v0 = 2 * a.n_kh * D + h * D + blk * kDB;

    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    float *Q = reinterpret_cast<float *>(smem + L::q);
    float *K = reinterpret_cast<float *>(smem + L::k);
    float *Kt = reinterpret_cast<float *>(smem + L::kt);
    float *Vb = reinterpret_cast<float *>(smem + L::vb);
    float *S = reinterpret_cast<float *>(smem + L::s);
    float *Tm = reinterpret_cast<float *>(smem + L::tm);
    float *Pm = reinterpret_cast<float *>(smem + L::pm);
    float *Yt = reinterpret_cast<float *>(smem + L::yt);
    float *Ut = reinterpret_cast<float *>(smem + L::ut);
    act_t *raw = reinterpret_cast<act_t *>(smem + L::tm);
    float *Gam = reinterpret_cast<float *>(smem + L::sc);  // Gamma_t
    float *gam = Gam + C;                                  // gamma_t = exp(Gamma_t)
    float *bet = gam + C;                                  // beta_t
    float *dec = bet + C;                                  // exp(Gamma_C - Gamma_t)

    const act_t *qkv = static_cast<const act_t *>(a.qkv);
    auto gchan = [&](int lc) -> int { return lc < D ? q0 + lc : (lc < 2 * D ? k0 + (lc - D) : v0 + (lc - 2 * D)); };
    auto to_f32 = [](act_t x) -> float {
        if constexpr (ACT_BF16)
            return bf16_to_f32(x);
        else
            return x;
    };

    // ---- the state block (rows blk*16 .. +16 of value head h) and the conv taps / conv state
    const float *st = a.state + ((size_t)a.slot * a.n_vh + h) * D * D + (size_t)blk * kDB * D;
    for (int i = tid; i < kDB * D / 4; i += kPThreads) reinterpret_cast<f4 *>(S)[i] = reinterpret_cast<const f4 *>(st)[i];
    constexpr int CPT = (NCH + kPThreads - 1) / kPThreads;
    f4 wv[CPT];
    float hist[CPT][3];  // conv window rows before the chunk (conv state for the first chunk)
    const float *cs = a.conv_state + (size_t)a.slot * 3 * Cc;
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
        const int lc = tid + j * kPThreads;
        if (lc < NCH) {
            const int gc = gchan(lc);
            wv[j] = *reinterpret_cast<const f4 *>(a.conv_w + (size_t)gc * 4);
#pragma unroll
            for (int r = 0; r < 3; ++r) hist[j][r] = cs[(size_t)r * Cc + gc];
        }
    }
    const float negA = -expf(a.A_log[h]), dtb = a.dt_bias[h];

    const int nchunks = (T + C - 1) / C;
#pragma unroll 1
    for (int c = 0; c < nchunks; ++c) {
        const int t0 = c * C;
        const int Lc = min(C, T - t0);  // valid tokens in this chunk
        // ================= stage the chunk's raw rows (tokens t0 .. t0+Lc-1) into LDS ============
        {
            constexpr int nvr = NCH / VEC;
            for (int it = tid; it < C * nvr; it += kPThreads) {
                const int r = it / nvr, lc = (it % nvr) * VEC;
                if (r < Lc)
                    lds_dma16(qkv + ((size_t)t0 + r) * Cc + gchan(lc), raw + it * VEC);
                else
                    *reinterpret_cast<f4 *>(raw + it * VEC) = f4{0.f, 0.f, 0.f, 0.f};
            }
        }
        float gl = 0.f, bl = 0.f;
        if (tid < Lc) {
            const size_t tok = ((size_t)t0 + tid) * a.n_vh + h;
            const float al = load_act<ACT_BF16>(a.alpha, tok);
            bl = load_act<ACT_BF16>(a.beta, tok);
            gl = negA * softplus_f(al + dtb);
        }
        __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0)
        // Gamma = inclusive prefix sum of g over the chunk (wave 0); padded tokens have g = 0, beta = 0
        if (wave == 0) {
            float x = gl;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float y = __shfl_up(x, off);
                if (lane >= off) x += y;
            }
            Gam[lane] = x;
            gam[lane] = expf(x);
            bet[lane] = bl;
            const float gC = __shfl(x, 63);
            dec[lane] = expf(gC - x);
        }
        __syncthreads();

        // ================= conv (one thread per channel) =================
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            const int lc = tid + j * kPThreads;
            if (lc < NCH) {
                const f4 w = wv[j];
                float x0 = hist[j][0], x1 = hist[j][1], x2 = hist[j][2];
                for (int t = 0; t < C; ++t) {
                    const float x3 = to_f32(raw[t * NCH + lc]);
                    float y = conv4(w, x0, x1, x2, x3);
                    if constexpr (QKN) y = y * sigmoid_f(y);
                    if (t >= Lc) y = 0.f;  // padded tokens contribute nothing
                    if (lc < D) {
                        Q[t * D + lc] = y;
                    } else if (lc < 2 * D) {
                        K[t * D + (lc - D)] = y;
                        Kt[(lc - D) * C + t] = y;
                    } else {
                        Vb[t * kDB + (lc - 2 * D)] = y;
                    }
                    // the window of the next chunk starts with this chunk's last three rows
                    if (t < Lc) {
                        x0 = x1;
                        x1 = x2;
                        x2 = x3;
                    }
                }
                hist[j][0] = x0;
                hist[j][1] = x1;
                hist[j][2] = x2;
            }
        }
        __syncthreads();
        if constexpr (QKN) {  // q, k scaled to unit length (+1e-6), q by d_k^-1/2; one wave per token
            for (int t = wave; t < Lc; t += kPThreads / 64) {
                constexpr int E = D / 64;
                float qv[E], kv[E], nq = 0.f, nk = 0.f;
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    qv[e] = Q[t * D + lane + 64 * e];
                    kv[e] = K[t * D + lane + 64 * e];
                    nq += qv[e] * qv[e];
                    nk += kv[e] * kv[e];
                }
                nq = wave_sum(nq);
                nk = wave_sum(nk);
                const float sq = 1.0f / sqrtf(nq + 1e-6f) / sqrtf((float)D);
                const float sk = 1.0f / sqrtf(nk + 1e-6f);
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    Q[t * D + lane + 64 * e] = qv[e] * sq;
                    K[t * D + lane + 64 * e] = kv[e] * sk;
                    Kt[(lane + 64 * e) * C + t] = kv[e] * sk;
                }
            }
            __syncthreads();
        }

        // ================= A = strictly-lower(beta_t e^{G_t-G_s} K K^T) into Tm  (MFMA) ===========
        // wave w: row tile w, column tiles 0..w; upper tiles are zero
        {
            const int w = wave;
            for (int ct = 0; ct < 4; ++ct) {
                f4 acc = {0.f, 0.f, 0.f, 0.f};
                if (ct <= w)
                    for (int k0 = 0; k0 < D; k0 += 32) acc = mma_tile<F32>(K, D, 16 * w, K, D, 16 * ct, k0, acc, lane);
                const int s_ = 16 * ct + (lane & 15);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 16 * w + (lane >> 4) * 4 + r;
                    Tm[t * C + s_] = (s_ < t) ? bet[t] * expf(Gam[t] - Gam[s_]) * acc[r] : 0.f;
                }
            }
        }
        __syncthreads();
        // ================= T = (I + A)^-1, blocked fp32 substitution =================
        // diagonal 16x16 blocks: wave w, lane c < 16 solves column c of (I + A_ww)^-1
        if (lane < 16) {
            const int w = wave, cc = lane;
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float acc = (r == cc) ? 1.f : 0.f;
#pragma unroll
                for (int s_ = 0; s_ < r; ++s_) acc -= Tm[(16 * w + r) * C + 16 * w + s_] * x[s_];
                x[r] = (r < cc) ? 0.f : acc;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) Tm[(16 * w + r) * C + 16 * w + cc] = x[r];
        }
        __syncthreads();
        // off-diagonal blocks, block row i = 1..3: T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj
        for (int i = 1; i < 4; ++i) {
            // X_ij (j < i) into the scratch Pm, one element per thread per pass
            for (int e = tid; e < i * 256; e += kPThreads) {
                const int j = e / 256, r = (e % 256) / 16, cc = e % 16;
                float acc = 0.f;
                for (int kb = j; kb < i; ++kb)
#pragma unroll
                    for (int m = 0; m < 16; ++m) acc += Tm[(16 * i + r) * C + 16 * kb + m] * Tm[(16 * kb + m) * C + 16 * j + cc];
                Pm[(16 * i + r) * C + 16 * j + cc] = acc;
            }
            __syncthreads();
            for (int e = tid; e < i * 256; e += kPThreads) {
                const int j = e / 256, r = (e % 256) / 16, cc = e % 16;
                float acc = 0.f;
#pragma unroll
                for (int m = 0; m < 16; ++m) acc += Tm[(16 * i + r) * C + 16 * i + m] * Pm[(16 * i + m) * C + 16 * j + cc];
                Tm[(16 * i + r) * C + 16 * j + cc] = -acc;
            }
            __syncthreads();
        }

        // ================= P = lower(e^{G_t-G_s} Q K^T) (MFMA), Y = beta V - beta gamma K S^T ======
        {
            const int w = wave;
            for (int ct = 0; ct < 4; ++ct) {
                f4 acc = {0.f, 0.f, 0.f, 0.f};
                if (ct <= w)
                    for (int k0 = 0; k0 < D; k0 += 32) acc = mma_tile<F32>(Q, D, 16 * w, K, D, 16 * ct, k0, acc, lane);
                const int s_ = 16 * ct + (lane & 15);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 16 * w + (lane >> 4) * 4 + r;
                    Pm[t * C + s_] = (s_ <= t) ? expf(Gam[t] - Gam[s_]) * acc[r] : 0.f;
                }
            }
            f4 acc = {0.f, 0.f, 0.f, 0.f};
            for (int k0 = 0; k0 < D; k0 += 32) acc = mma_tile<F32>(K, D, 16 * w, S, D, 0, k0, acc, lane);
            const int i = lane & 15;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * w + (lane >> 4) * 4 + r;
                Yt[i * C + t] = bet[t] * (Vb[t * kDB + i] - gam[t] * acc[r]);
            }
        }
        __syncthreads();
        // ================= U = T Y (MFMA) =================
        {
            const int w = wave;
            f4 acc = {0.f, 0.f, 0.f, 0.f};
            for (int k0 = 0; k0 < C; k0 += 32) acc = mma_tile<F32>(Tm, C, 16 * w, Yt, C, 0, k0, acc, lane);
            const int i = lane & 15;
#pragma unroll
            for (int r = 0; r < 4; ++r) Ut[i * C + 16 * w + (lane >> 4) * 4 + r] = acc[r];
        }
        __syncthreads();
        // ================= O = diag(gamma) Q S^T + P U ;  S' = gamma_C S + U^T diag(dec) K ==========
        f4 snew[2];
        {
            const int w = wave;
            f4 acc = {0.f, 0.f, 0.f, 0.f};
            for (int k0 = 0; k0 < D; k0 += 32) acc = mma_tile<F32>(Q, D, 16 * w, S, D, 0, k0, acc, lane);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] *= gam[16 * w + (lane >> 4) * 4 + r];
            for (int k0 = 0; k0 < C; k0 += 32) acc = mma_tile<F32>(Pm, C, 16 * w, Ut, C, 0, k0, acc, lane);
            const int i = lane & 15;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * w + (lane >> 4) * 4 + r;
                if (t < Lc) a.o_ws[(((size_t)t0 + t) * a.n_vh + h) * D + blk * kDB + i] = acc[r];
            }
            // S' block: rows i = 4*(lane>>4)+r, columns j = 16*ct + (lane&15), ct = 2w, 2w+1
            const float gC = gam[Lc - 1];
#pragma unroll
            for (int q2 = 0; q2 < 2; ++q2) {
                const int ct = 2 * w + q2;
                if (ct * 16 >= D) {
                    snew[q2] = f4{0.f, 0.f, 0.f, 0.f};
                    continue;
                }
                f4 sa;
#pragma unroll
                for (int r = 0; r < 4; ++r) sa[r] = gC * S[((lane >> 4) * 4 + r) * D + 16 * ct + (lane & 15)];
                for (int k0 = 0; k0 < C; k0 += 32) {
                    float av[8], bv[8];
                    load8(Ut + (lane & 15) * C + k0 + (lane >> 4) * 8, av);
                    load8(Kt + (16 * ct + (lane & 15)) * C + k0 + (lane >> 4) * 8, bv);
#pragma unroll
                    for (int e = 0; e < 8; ++e) bv[e] *= dec[k0 + (lane >> 4) * 8 + e];
                    sa = mma8<F32>(av, bv, sa);
                }
                snew[q2] = sa;
            }
        }
        __syncthreads();
        {
            const int w = wave;
#pragma unroll
            for (int q2 = 0; q2 < 2; ++q2) {
                const int ct = 2 * w + q2;
                if (ct * 16 < D)
#pragma unroll
                    for (int r = 0; r < 4; ++r) S[((lane >> 4) * 4 + r) * D + 16 * ct + (lane & 15)] = snew[q2][r];
            }
        }
        __syncthreads();
    }
    // ---- the state block after the last token
    float *sd = a.state + ((size_t)a.slot * a.n_vh + h) * D * D + (size_t)blk * kDB * D;
    for (int i = tid; i < kDB * D / 4; i += kPThreads) reinterpret_cast<f4 *>(sd)[i] = reinterpret_cast<const f4 *>(S)[i];
}

// out = o / sqrt(mean(o^2) + eps) * norm_w * silu(z) per (token, head); 16 lanes per row.  The
// conv state after the last token is written by the first rows' threads.
template <int D, bool ACT_BF16, bool OUT_BF16>
__global__ __launch_bounds__(256) void prefill_norm_kernel(PrefillArgs a)
{
    constexpr int EPL = D / 16;
    const int row = blockIdx.x * 16 + (threadIdx.x >> 4);
    const int cg = threadIdx.x & 15;
    const int nrows = a.T * a.n_vh;
    if (row < nrows) {
        const float *o = a.o_ws + (size_t)row * D + cg * EPL;
        float ov[EPL], ss = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            ov[e] = o[e];
            ss += ov[e] * ov[e];
        }
        ss = row16_sum(ss);
        const float inv = 1.0f / sqrtf(ss / (float)D + a.eps);
        const size_t base = (size_t)row * D + cg * EPL;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            const float zz = load_act<ACT_BF16>(a.z, base + e);
            const float y = ov[e] * inv * a.norm_w[cg * EPL + e] * (zz * sigmoid_f(zz));
            if constexpr (OUT_BF16)
                static_cast<uint16_t *>(a.out)[base + e] = f32_to_bf16(y);
            else
                static_cast<float *>(a.out)[base + e] = y;
        }
    } else {
        // conv state after the last token = the last three rows of concat(old conv state, qkv);
        // one thread per channel, in the row-groups after the token rows
        const int gc = (row - nrows) * 16 + cg;
        if (gc < a.C) {
            float r3[3];
#pragma unroll
            for (int r = 0; r < 3; ++r) {
                const int src = a.T + r;  // row of concat(conv state, qkv)
                r3[r] = src < 3 ? a.conv_state[((size_t)a.slot * 3 + src) * a.C + gc]
                                : load_act<ACT_BF16>(a.qkv, (size_t)(src - 3) * a.C + gc);
            }
#pragma unroll
            for (int r = 0; r < 3; ++r) a.conv_state[((size_t)a.slot * 3 + r) * a.C + gc] = r3[r];
        }
    }
}

size_t prefill_workspace_bytes(int d, int n_vh, int T) { return sizeof(float) * (size_t)T * n_vh * d; }

size_t prefill_lds_bytes(int d, bool act_bf16)
{
    if (d == 128) return act_bf16 ? PrefillLds<128, uint16_t>::total : PrefillLds<128, float>::total;
    return act_bf16 ? PrefillLds<64, uint16_t>::total : PrefillLds<64, float>::total;
}

template <int D, bool AB, bool OB, bool QKN>
static hipError_t launch_prefill_t(const PrefillArgs &a, hipStream_t stream)
{
    const size_t lds = prefill_lds_bytes(D, AB);
    hipLaunchKernelGGL((prefill_chunk_kernel<D, AB, QKN>), dim3(a.n_vh * (D / kDB)), dim3(kPThreads), lds, stream, a);
    if (hipError_t e = hipGetLastError()) return e;
    const long rows = (long)a.T * a.n_vh;
    const long conv_rows = (a.C + 15) / 16;  // 16 threads per row-group also cover the conv state
    hipLaunchKernelGGL((prefill_norm_kernel<D, AB, OB>), dim3((unsigned)((rows + conv_rows + 15) / 16)), dim3(256), 0,
                       stream, a);
    return hipGetLastError();
}
template <int D, bool AB, bool OB>
static hipError_t launch_prefill_q(const PrefillArgs &a, const LaunchCfg &c, hipStream_t s)
{
    return c.qk_norm ? launch_prefill_t<D, AB, OB, true>(a, s) : launch_prefill_t<D, AB, OB, false>(a, s);
}
template <int D, bool AB>
static hipError_t launch_prefill_o(const PrefillArgs &a, const LaunchCfg &c, hipStream_t s)
{
    return c.out_bf16 ? launch_prefill_q<D, AB, true>(a, c, s) : launch_prefill_q<D, AB, false>(a, c, s);
}
template <int D>
static hipError_t launch_prefill_a(const PrefillArgs &a, const LaunchCfg &c, hipStream_t s)
{
    return c.act_bf16 ? launch_prefill_o<D, true>(a, c, s) : launch_prefill_o<D, false>(a, c, s);
}

hipError_t launch_prefill(const PrefillArgs &a, const LaunchCfg &c, hipStream_t stream)
{
    if (a.d == 128) return launch_prefill_a<128>(a, c, stream);
    if (a.d == 64) return launch_prefill_a<64>(a, c, stream);
    return hipErrorInvalidValue;
}

}  // namespace gdn
