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
// Everything that does not depend on S (conv, gates, A -> T, P) is the same for every value-row
// block and every chunk can compute it at once, so it runs first, chunk-parallel; only Y, U, O
// and S' remain on the sequential chain of chunks.
// Kernel 1 (prep): one workgroup per (chunk, key head): conv of the chunk's q | k channels and the
// Gram products K K^T and Q K^T on MFMA, shared by the key head's value heads; then per value head
// the gates, A and P, and T by blocked fp32 forward substitution.  It writes the operands of the
// scan to the workspace as LDS images (the layouts the scan reads), so the scan copies them with
// flat global_load_lds transfers.
// Kernel 2 (scan): one workgroup per (value head, block of 16 value rows).  Rows of S are
// independent given the keys, so the blocks never communicate; each walks the chunks in order,
// convolving its own v channels and keeping its S block in fp32 registers (LDS holds only its
// MFMA operand form) while the next chunk's operands travel in.  Dense products run on
// v_mfma_f32_16x16x32_bf16 with each fp32 operand split into bf16 hi + lo parts (a b ~ a_hi b_hi +
// a_hi b_lo + a_lo b_hi, ~2^-16 relative), so the fp32 state is not rounded to bf16; with fp32
// activations the products run on the fp32 MFMA.
// Kernel 3 (epilogue): RMS norm over d_v + SiLU(z) gate of every token (the d_v blocks of kernel 2
// meet here through an fp32 workspace), and the conv state after the last token.
#include "gdn_device.h"
#include "gdn_internal.h"

#include <type_traits>

namespace gdn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kChunk = 64;  // tokens per chunk
// Value rows per scan workgroup (16-row MFMA tiles).  The scan's step is bound by moving each
// chunk's q, k, T and P images into the workgroup, the same bytes whatever its share of rows, so
// the rows are spread as thin as keeps the chip busy: 16 rows give 8 workgroups per d=128 head,
// 256 for 32 heads, one per CU (32 rows: 128 workgroups, 7% slower over the whole prefill).
constexpr int kSR = 16;
constexpr int kRT = kSR / 16;  // row tiles per scan workgroup
static_assert(kRT == 1 || kRT == 2, "one or two 16-row tiles");
constexpr int kPThreads = 256;
constexpr int kCP = kChunk + 4;  // padded row stride of the chunk x chunk matrices

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

// Transposing 64-bit LDS load (ds_read_b64_tr_b16).  In every group of 16 lanes, lane i receives
// element i % 4 of the 4-element chunks that lanes i / 4, i / 4 + 4, i / 4 + 8 and i / 4 + 12 of
// the group address, in that order.  So when lane 4 j + q of a group points at row r0 + j, columns
// c0 + 4 q .. c0 + 4 q + 3 of a row-major bf16 matrix, lane i of the group gets column c0 + i,
// rows r0 .. r0 + 3: four consecutive k values of a column, as an MFMA operand wants them.
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_tr;
typedef unsigned long long u64x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ unsigned long long lds_load_tr4(const __bf16 *p)
{
#if defined(__HIP_DEVICE_COMPILE__)
    const auto lp = (__attribute__((address_space(3))) bf16x4_tr *)(const_cast<__bf16 *>(p));
    return __builtin_bit_cast(unsigned long long, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(lp));
#else
    (void)p;
    return 0;
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

// 16x16 fp32 block product on the fp32 MFMA: acc += X(16x16 at ld, rows r0, cols c0) *
// Y(16x16, rows k0.., cols n0..), both in kCP-padded LDS matrices.  Lane l supplies X[l%16][4s + l/16]
// and Y[4s + l/16][l%16] for step s; the result is in the usual layout (rows 4 (l/16) + i, col l%16).
__device__ __forceinline__ f4 blk16(const float *X, int xr0, int xc0, const float *Y, int yr0, int yc0, f4 acc,
                                    int lane)
{
#pragma unroll
    for (int st = 0; st < 4; ++st) {
        const int kk = 4 * st + (lane >> 4);
        acc = mfma4f32(X[(xr0 + (lane & 15)) * kCP + xc0 + kk], Y[(yr0 + kk) * kCP + yc0 + (lane & 15)], acc);
    }
    return acc;
}


// ---- MFMA operand matrices shared by the prep (as images it writes) and the scan (in LDS) ----
// One lane's 8 consecutive k values of an MFMA operand: fp32 values for the fp32 MFMA, or the bf16
// hi and lo parts of the fp32 values for the bf16 MFMA.
template <bool F32>
struct Frag;
template <>
struct Frag<true> {
    float v[8];
};
template <>
struct Frag<false> {
    bf16x8 hi, lo;
};

// One 32-deep step of a 16x16 product.  Lane l holds a = A[l % 16][8 (l / 16) + e] and
// b = B[8 (l / 16) + e][l % 16], e = 0 .. 7, of the 16x32 and 32x16 operands; the result rows are
// 4 (l / 16) + r, columns l % 16.
// F32: eight v_mfma_f32_16x16x4_f32, step e taking k index 8 kk + e for the instruction's kk = l / 16
// (fp32 products, the precision of the all-fp32 path).  Otherwise one 16x16x32 bf16 MFMA per
// pair of bf16 parts: a b ~ a_lo b_hi + a_hi b_lo + a_hi b_hi (the a_lo b_lo term, ~2^-16 of a b,
// is dropped), smallest terms first.
template <bool F32>
__device__ __forceinline__ f4 mma(const Frag<F32> &a, const Frag<F32> &b, f4 acc)
{
    if constexpr (F32) {
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = mfma4f32(a.v[e], b.v[e], acc);
    } else {
        acc = mfma16(a.lo, b.hi, acc);
        acc = mfma16(a.hi, b.lo, acc);
        acc = mfma16(a.hi, b.hi, acc);
    }
    return acc;
}

// N independent products acc[n] += a[n] b[n], issued term by term across n, so that consecutive
// MFMAs never depend on each other (a dependent MFMA waits for its predecessor to finish).  Each
// accumulator sees exactly the term order of mma().
template <bool F32, int N>
__device__ __forceinline__ void mma_n(const Frag<F32> (&a)[N], const Frag<F32> (&b)[N], f4 (&acc)[N])
{
    if constexpr (F32) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
#pragma unroll
            for (int n = 0; n < N; ++n) acc[n] = mfma4f32(a[n].v[e], b[n].v[e], acc[n]);
    } else {
#pragma unroll
        for (int n = 0; n < N; ++n) acc[n] = mfma16(a[n].lo, b[n].hi, acc[n]);
#pragma unroll
        for (int n = 0; n < N; ++n) acc[n] = mfma16(a[n].hi, b[n].lo, acc[n]);
#pragma unroll
        for (int n = 0; n < N; ++n) acc[n] = mfma16(a[n].hi, b[n].hi, acc[n]);
    }
}

// A [ROWS][COLS] fp32 matrix kept ready for MFMA operand loads: fp32 (F32), or already split into a
// bf16 hi plane followed by a bf16 lo plane (both the size of the fp32 matrix together).  Groups
// of 8 consecutive columns are XOR-swizzled by the row, so the 16 rows one operand load touches
// spread over the LDS banks.  The same layout serves as the prep's workspace image and the scan's
// LDS copy, so moving it is a flat copy.
template <bool F32, int ROWS, int COLS>
struct Mat {
    static constexpr int NG = COLS / 8;
    static constexpr int floats = ROWS * COLS;  // size in floats either way
    __device__ static int idx(int r, int c) { return r * COLS + ((((c >> 3) ^ r) & (NG - 1)) << 3) + (c & 7); }
    // operand fragment: row r, columns c0 .. c0 + 7 (c0 a multiple of 8)
    __device__ static Frag<F32> load(const float *m, int r, int c0)
    {
        Frag<F32> f;
        if constexpr (F32) {
            load8(m + idx(r, c0), f.v);
        } else {
            const __bf16 *hp = reinterpret_cast<const __bf16 *>(m);
            f.hi = *reinterpret_cast<const bf16x8 *>(hp + idx(r, c0));
            f.lo = *reinterpret_cast<const bf16x8 *>(hp + ROWS * COLS + idx(r, c0));
        }
        return f;
    }
    // operand fragment down a column (bf16 planes only): lane li of its 16-lane group gets column
    // c0 + li, rows r0 .. r0 + 7 (r0 the same for the group, c0 a multiple of 8), by two transposing
    // loads per plane
    __device__ static Frag<F32> load_col(const float *m, int r0, int c0, int li)
    {
        static_assert(!F32, "transposing loads move 16-bit elements");
        const __bf16 *hp = reinterpret_cast<const __bf16 *>(m);
        const int r = r0 + (li >> 2), c = c0 + 4 * (li & 3);
        const int a0 = idx(r, c), a1 = idx(r + 4, c);
        Frag<F32> f;
        f.hi = __builtin_bit_cast(bf16x8, u64x2{lds_load_tr4(hp + a0), lds_load_tr4(hp + a1)});
        f.lo = __builtin_bit_cast(bf16x8, u64x2{lds_load_tr4(hp + ROWS * COLS + a0), lds_load_tr4(hp + ROWS * COLS + a1)});
        return f;
    }
    // element (r, c) into fragment slot e (gathers down a column)
    __device__ static void get(const float *m, int r, int c, Frag<F32> &f, int e)
    {
        if constexpr (F32) {
            f.v[e] = m[idx(r, c)];
        } else {
            const __bf16 *hp = reinterpret_cast<const __bf16 *>(m);
            f.hi[e] = hp[idx(r, c)];
            f.lo[e] = hp[ROWS * COLS + idx(r, c)];
        }
    }
    __device__ static void put(float *m, int r, int c, float x)
    {
        if constexpr (F32) {
            m[idx(r, c)] = x;
        } else {
            __bf16 *hp = reinterpret_cast<__bf16 *>(m);
            const __bf16 h = (__bf16)x;
            hp[idx(r, c)] = h;
            hp[ROWS * COLS + idx(r, c)] = (__bf16)(x - (float)h);
        }
    }
    // four consecutive columns c0 .. c0 + 3 of row r (c0 a multiple of 4): one 8-byte store per
    // bf16 plane, or one 16-byte store of fp32
    __device__ static void put4(float *m, int r, int c0, f4 x)
    {
        if constexpr (F32) {
            *reinterpret_cast<f4 *>(m + idx(r, c0)) = x;
        } else {
            uint32_t h[2], l[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const __bf16 h0 = (__bf16)x[2 * j], h1 = (__bf16)x[2 * j + 1];
                const __bf16 l0 = (__bf16)(x[2 * j] - (float)h0), l1 = (__bf16)(x[2 * j + 1] - (float)h1);
                h[j] = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
                l[j] = (uint32_t)__builtin_bit_cast(uint16_t, l0) | ((uint32_t)__builtin_bit_cast(uint16_t, l1) << 16);
            }
            __bf16 *hp = reinterpret_cast<__bf16 *>(m);
            *reinterpret_cast<uint2 *>(hp + idx(r, c0)) = uint2{h[0], h[1]};
            *reinterpret_cast<uint2 *>(hp + ROWS * COLS + idx(r, c0)) = uint2{l[0], l[1]};
        }
    }
    __device__ static void put8(float *m, int r, int c0, const float (&x)[8])
    {
        if constexpr (F32) {
            *reinterpret_cast<f4 *>(m + idx(r, c0)) = f4{x[0], x[1], x[2], x[3]};
            *reinterpret_cast<f4 *>(m + idx(r, c0) + 4) = f4{x[4], x[5], x[6], x[7]};
        } else {
            bf16x8 hi, lo;
            split8(x, hi, lo);
            __bf16 *hp = reinterpret_cast<__bf16 *>(m);
            *reinterpret_cast<bf16x8 *>(hp + idx(r, c0)) = hi;
            *reinterpret_cast<bf16x8 *>(hp + ROWS * COLS + idx(r, c0)) = lo;
        }
    }
};

// A 64 x 64 lower-triangular operand (T or P) without its upper-right 32 x 32 block, which is all
// zero: block L = rows 0..63 x columns 0..31, then block R = rows 32..63 x columns 32..63, each a
// Mat image.  12 KiB instead of 16 per image, in the workspace and in LDS.
template <bool F32>
struct Tri {
    using ML = Mat<F32, kChunk, kChunk / 2>;
    using MR = Mat<F32, kChunk / 2, kChunk / 2>;
    static constexpr int floats = ML::floats + MR::floats;
    // row r, columns c0 .. c0 + 7 (c0 a multiple of 8, not in the zero block)
    __device__ static Frag<F32> load(const float *m, int r, int c0)
    {
        return c0 < kChunk / 2 ? ML::load(m, r, c0) : MR::load(m + ML::floats, r - kChunk / 2, c0 - kChunk / 2);
    }
    // row r, columns c0 .. c0 + 7; nothing is stored for the zero block
    __device__ static void put8(float *m, int r, int c0, const float (&x)[8])
    {
        if (c0 < kChunk / 2)
            ML::put8(m, r, c0, x);
        else if (r >= kChunk / 2)
            MR::put8(m + ML::floats, r - kChunk / 2, c0 - kChunk / 2, x);
    }
};

// Workspace (floats), nc = number of chunks:
//   o  [nc * 64][H_v][d]         fp32 readout before the norm (whole chunks: the tail is scratch)
//   qk [nc][H_k][2][64 * d]      conv'd q then k of the chunk, per key head
// (q, k, T and P as Mat images: fp32, or split into bf16 hi / lo planes for bf16 activations)
//   t  [nc][H_v][3072]           T = (I + A)^-1   (Tri images: the zero upper-right block left out)
//   p  [nc][H_v][3072]           P
//   g  [nc][H_v][256]            gamma | beta | exp(Gamma_C - Gamma) | 0, 64 each
// (the scan convolves v itself from the raw activations)
constexpr int kGateRec = 4 * kChunk;
constexpr int kTriFloats = kChunk * kChunk / 2 + kChunk * kChunk / 4;  // a Tri image
struct PrefillWs {
    size_t o, qk, t, p, g, total;
};
__host__ __device__ inline PrefillWs prefill_ws(int d, int n_kh, int n_vh, int T)
{
    const size_t nc = ((size_t)T + kChunk - 1) / kChunk;
    PrefillWs w;
    w.o = 0;
    w.qk = w.o + nc * kChunk * n_vh * d;
    w.t = w.qk + nc * n_kh * 2 * kChunk * d;
    w.p = w.t + nc * n_vh * kTriFloats;
    w.g = w.p + nc * n_vh * kTriFloats;
    w.total = w.g + nc * n_vh * kGateRec;
    return w;
}

template <int D>
struct PrepLds {
    static constexpr int C = kChunk;
    // q and k are convolved in NH passes over their channels, D / NH channels in LDS at a time, so
    // that three d = 128 workgroups share a CU (their phases are latency-bound: more of them hide it)
    static constexpr int NH = D == 128 ? 2 : 1;
    static constexpr int DH = D / NH;
    static constexpr size_t qk_bytes = sizeof(float) * 2 * C * DH;
    static constexpr size_t tp_bytes = sizeof(float) * (2 * C * kCP + 4 * 256);
    static constexpr size_t q = 0;                               // [C][DH] as a Mat image
    static constexpr size_t k = q + sizeof(float) * C * DH;      // [C][DH] as a Mat image
    static constexpr size_t tm = 0;                              // once q, k are consumed: [C][kCP] A, then T
    static constexpr size_t pm = tm + sizeof(float) * C * kCP;   //                         [C][kCP] P
    static constexpr size_t scr = pm + sizeof(float) * C * kCP;  //                         [4][16][16] scratch
    static constexpr int heads = 4;  // value heads whose gates are resident at once
    static constexpr size_t gate = qk_bytes > tp_bytes ? qk_bytes : tp_bytes;  // per head: Gamma (fp64), gamma, beta, decay
    static constexpr int slot_floats = 5 * C;  // Gamma as C doubles, then gamma, beta, decay [3][C]
    static constexpr size_t total = gate + sizeof(float) * heads * slot_floats;
};
static_assert(3 * PrepLds<128>::total <= 160 * 1024 && 3 * PrepLds<64>::total <= 160 * 1024,
              "three prep workgroups must fit one CU's LDS");

// Scan workgroup: kSR value rows of one value head.  Its LDS, in bytes:
template <int D, bool ACT_BF16>
struct ScanLds {
    static constexpr int C = kChunk;
    static constexpr size_t kimg = sizeof(float) * C * D;     // a q or k image
    static constexpr size_t timg = sizeof(float) * kTriFloats;  // a T or P image
    // raw v rows of the block's kSR channels, window rows 0 .. C + 2 (token t0 - 3 + row), moved
    // 1 KiB (one 64-lane 16-byte transfer) at a time
    static constexpr int vrow = kSR * (ACT_BF16 ? 2 : 4);  // bytes per row
    static constexpr int vrows_per_dma = 1024 / vrow;
    static constexpr int vdmas = (C + 3 + vrows_per_dma - 1) / vrows_per_dma;
    static constexpr size_t vimg = 1024 * vdmas;
    static constexpr size_t gimg = sizeof(float) * kGateRec;
    static constexpr size_t kb = 0;                          // k image of the chunk in progress
    static constexpr size_t q = kb + kimg;                   // [2] q images (chunk parity)
    static constexpr size_t tm = q + 2 * kimg;               // T image
    static constexpr size_t pm = tm + timg;                  // [2] P images (chunk parity)
    static constexpr size_t vb = pm + 2 * timg;              // raw v rows
    static constexpr size_t gb = vb + vimg;                  // [2] gate records (chunk parity)
    static constexpr size_t yp = gb + 2 * gimg;              // Y^T [kSR][C]  (operand form)
    static constexpr size_t up = yp + sizeof(float) * kSR * C;  // U^T [kSR][C]  (operand form)
    // U^T diag(dec) [kSR][C] (operand form; bf16 only: fp32 operands are scaled where they are read)
    static constexpr size_t dp = up + sizeof(float) * kSR * C;
    static constexpr size_t sx = dp + (ACT_BF16 ? sizeof(float) * kSR * C : 0);  // S [kSR][D] (operand form)
    static constexpr size_t touch = sx + sizeof(float) * kSR * D;  // where the L2 touches land (never read)
    static constexpr size_t total = touch + 256;
};
static_assert(ScanLds<128, true>::total <= 160 * 1024 && ScanLds<128, false>::total <= 160 * 1024,
              "the d=128 scan must fit one CU's LDS");

// e^x for a decay ratio (x = Gamma_t - Gamma_s <= 0): v_exp_f32 of x log2(e), two instructions
// against the ~13 of the fully range-reduced expf.  Rounding the product costs a relative error of
// about |x| 2^-24, below 1e-6 wherever e^x exceeds 1e-7; ratios far below the fp32 range come out
// as 0, where they scale O(1) Gram entries down to nothing either way.
__device__ __forceinline__ float exp_decay(float x) { return __builtin_amdgcn_exp2f(x * 1.44269504088896341f); }

// ============================== kernel 1: per (chunk, key head) ==============================
// The q | k conv and the Gram products K K^T and Q K^T are shared by the key head's value heads;
// the gates, A / P, T and the v conv are per value head, in a loop.
template <int D, bool ACT_BF16, bool QKN>
__global__ __launch_bounds__(kPThreads) __attribute__((amdgpu_waves_per_eu(3, 3))) void prefill_prep_kernel(PrefillArgs a)
{
    using act_t = typename std::conditional<ACT_BF16, uint16_t, float>::type;
    using L = PrepLds<D>;
    constexpr bool F32 = !ACT_BF16;
    constexpr int C = kChunk;
    constexpr int QKG = 2 * D / 4;  // q | k channel groups of 4 (one per lane of a conv wave)
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int R = a.n_vh / a.n_kh;

    const int c = blockIdx.x / a.n_kh, hk = blockIdx.x % a.n_kh;
    const int T = a.T;
    const int Cc = a.C;  // conv channels
    const int t0 = c * C, Lc = min(C, T - t0);
    const int q0 = hk * D, k0 = a.n_kh * D + hk * D;
    const PrefillWs w = prefill_ws(D, a.n_kh, a.n_vh, T);

    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    float *Q = reinterpret_cast<float *>(smem + L::q);
    float *K = reinterpret_cast<float *>(smem + L::k);
    float *Tm = reinterpret_cast<float *>(smem + L::tm);
    float *Pm = reinterpret_cast<float *>(smem + L::pm);
    // gates of value head hk R + hh, kept in slot hh % L::heads: Gamma_t (fp64), then gamma_t =
    // exp(Gamma_t), beta_t (0 past the end), exp(Gamma_C - Gamma_t) (fp32).  Gamma is a running sum
    // of log decays that reaches hundreds within a chunk under strong decay, where an fp32 ulp
    // (~6e-5 at 650) would leave the ratios exp(Gamma_t - Gamma_s) of nearby tokens that relative
    // error; its differences are taken in fp64 and only then rounded.
    auto gate_slot = [&](int hh) { return reinterpret_cast<float *>(smem + L::gate) + (hh % L::heads) * L::slot_floats; };

    const act_t *qkv = static_cast<const act_t *>(a.qkv);
    auto gchan = [&](int lc) -> int { return lc < D ? q0 + lc : k0 + (lc - D); };
    // Rows are loaded raw (every load of a conv issued before any is used) and converted after:
    // channels lc .. lc+3 of token t0 + t; before the first chunk the three rows at t < 0 come
    // from the conv state (fp32) instead.
    using raw4 = typename std::conditional<ACT_BF16, uint2, f4>::type;
    auto ld_raw = [&](int t, int lc) -> raw4 {
        return *reinterpret_cast<const raw4 *>(qkv + ((size_t)t0 + t) * Cc + gchan(lc));
    };
    auto cvt = [](raw4 u) -> f4 {
        if constexpr (ACT_BF16)
            return f4{bf16_to_f32((uint16_t)(u.x & 0xffffu)), bf16_to_f32((uint16_t)(u.x >> 16)),
                      bf16_to_f32((uint16_t)(u.y & 0xffffu)), bf16_to_f32((uint16_t)(u.y >> 16))};
        else
            return u;
    };
    auto hist4 = [&](int t, int lc) -> f4 {  // -3 <= t < 0, first chunk only
        return *reinterpret_cast<const f4 *>(a.conv_state + ((size_t)a.slot * 3 + 3 + t) * Cc + gchan(lc));
    };
    const int tmin = c == 0 ? 0 : -3;  // lowest row of qkv a conv may read

    // Gate inputs of value head hk R + hh at this lane's token.  The loads are unconditional (a lane
    // past the chunk or a head past R reads a valid entry it discards) and raw, so that nothing
    // computed from them makes the compiler wait for them where they are issued.
    using word_t = typename std::conditional<ACT_BF16, uint16_t, uint32_t>::type;  // bf16 or fp32 bits
    struct GateIn {
        uint32_t al, be;
        float alog, dtb;
    };
    auto gate_load = [&](int hh) -> GateIn {
        const int h = hk * R + min(hh, R - 1);
        const size_t e = ((size_t)t0 + min(lane, Lc - 1)) * a.n_vh + h;
        return GateIn{static_cast<const word_t *>(a.alpha)[e], static_cast<const word_t *>(a.beta)[e], a.A_log[h],
                      a.dt_bias[h]};
    };
    auto word_f32 = [](uint32_t u) -> float {
        if constexpr (ACT_BF16)
            return bf16_to_f32((uint16_t)u);
        else
            return __builtin_bit_cast(float, u);
    };
    // one wave: Gamma = prefix sum of g; padded tokens get g = 0, beta = 0
    auto gate_put = [&](int hh, const GateIn &in) {
        float g = 0.f, b = 0.f;
        if (lane < Lc) {
            g = -expf(in.alog) * softplus_f(word_f32(in.al) + in.dtb);
            b = word_f32(in.be);
        }
        double x = g;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const double y = __shfl_up(x, off);
            if (lane >= off) x += y;
        }
        reinterpret_cast<double *>(gate_slot(hh))[lane] = x;
        float *G = gate_slot(hh) + 2 * C;
        G[lane] = (float)exp(x);  // fp64 exponentials of fp64 sums, rounded once: 64 per head
        G[C + lane] = b;
        G[2 * C + lane] = (float)exp(__shfl(x, 63) - x);
    };

    // the first value heads' gate inputs travel with the q | k rows below
    GateIn gin = gate_load(wave);

    // ---- conv of q | k into LDS and into the scan's q and k images.  Every row a lane reads is
    // loaded before the first tap sum; the image stores go out as the values are formed, so they
    // travel while the conv and the Gram products run.  LDS holds q and k in operand form (bf16 hi /
    // lo planes), so the Gram products split nothing.
    constexpr int NH = L::NH, DH = L::DH;
    using MQ = Mat<F32, C, D>;   // the scan's q / k images
    using MH = Mat<F32, C, DH>;  // this pass's channels of q and k in LDS
    float *const qdst = a.ws + w.qk + ((size_t)c * a.n_kh + hk) * 2 * C * D;

    // The lower 16 x 16 tiles of K K^T (waves 0, 1) and Q K^T (waves 2, 3), accumulated in registers
    // pass by pass (MFMA; row tiles {0,3} or {1,2}: 5 tiles per wave), the k index in increasing
    // order over the passes.  Each value head's A = strictly-lower(beta e^{G_t-G_s} K K^T) and
    // P = lower(e^{G_t-G_s} Q K^T) scale them.
    const int pair = wave & 1;
    auto tile_rt = [&](int jt) { return pair == 0 ? (jt == 0 ? 0 : 3) : (jt < 2 ? 1 : 2); };
    auto tile_ct = [&](int jt) { return pair == 0 ? (jt == 0 ? 0 : jt - 1) : (jt < 2 ? jt : jt - 2); };
    f4 tiles[5];
#pragma unroll
    for (int jt = 0; jt < 5; ++jt) tiles[jt] = f4{0.f, 0.f, 0.f, 0.f};
    auto gram = [&]() {
        const float *Am = wave < 2 ? K : Q;
#pragma unroll
        for (int jt = 0; jt < 5; ++jt) {
            // pair 0: (0,0) (3,0) (3,1) (3,2) (3,3);  pair 1: (1,0) (1,1) (2,0) (2,1) (2,2)
            const int rt = tile_rt(jt), ct = tile_ct(jt);
#pragma unroll
            for (int kk = 0; kk < DH; kk += 32) {
                const Frag<F32> fa = MH::load(Am, 16 * rt + (lane & 15), kk + (lane >> 4) * 8);
                const Frag<F32> fb = MH::load(K, 16 * ct + (lane & 15), kk + (lane >> 4) * 8);
                tiles[jt] = mma<F32>(fa, fb, tiles[jt]);
            }
        }
    };

    if constexpr (NH == 1) {
        // wave w takes tokens 16w .. 16w+15, a lane 4 channels
        if (lane < QKG) {
            const int lc = 4 * lane;
            const bool isq = lc < D;
            float *M = isq ? Q : K;
            float *img = isq ? qdst : qdst + C * D;
            const int mc = isq ? lc : lc - D;
            f4 wqk[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) wqk[j] = *reinterpret_cast<const f4 *>(a.conv_w + (size_t)gchan(lc + j) * 4);
            raw4 rw[19];
#pragma unroll
            for (int i = 0; i < 19; ++i) rw[i] = ld_raw(min(max(16 * wave - 3 + i, tmin), Lc - 1), lc);
            const bool head_rows = c == 0 && wave == 0;  // the wave's first three rows precede the call
            f4 hs[3] = {};
            if (head_rows)
#pragma unroll
                for (int i = 0; i < 3; ++i) hs[i] = hist4(i - 3, lc);
            f4 xs[19];
#pragma unroll
            for (int i = 0; i < 19; ++i) xs[i] = (i < 3 && head_rows) ? hs[i < 3 ? i : 0] : cvt(rw[i]);
#pragma unroll
            for (int tt = 0; tt < 16; ++tt) {
                const int t = 16 * wave + tt;
                f4 y;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    float v = conv4(wqk[j], xs[tt][j], xs[tt + 1][j], xs[tt + 2][j], xs[tt + 3][j]);
                    if constexpr (QKN) v = v * sigmoid_f(v);
                    y[j] = t < Lc ? v : 0.f;
                }
                if constexpr (QKN) {  // unit length (+1e-6) over the head's channels; q also / sqrt(d)
                    float ss = y[0] * y[0] + y[1] * y[1] + y[2] * y[2] + y[3] * y[3];
                    ss = row16_sum(ss);
                    if constexpr (D == 128) ss += __shfl_xor(ss, 16);
                    const float sc = rsqrt_f(ss + 1e-6f) * (isq ? 1.0f / sqrtf((float)D) : 1.0f);
#pragma unroll
                    for (int j = 0; j < 4; ++j) y[j] *= sc;
                }
                MH::put4(M, t, mc, y);
                MQ::put4(img, t, mc, y);
            }
        }
        asm volatile("" : "+v"(gin.al), "+v"(gin.be), "+v"(gin.alog), "+v"(gin.dtb));  // loaded by now
        if (wave < min(R, L::heads)) gate_put(wave, gin);
        lds_barrier();  // q, k and the first heads' gates are in LDS
        gram();
    } else {
        // Two passes over the channel halves.  Wave w takes tokens 16w .. 16w+15, 8 per half wave
        // (th), a lane 4 channels of each half: q channels 4g .. 4g+3 (g < 16) or k channels
        // 4(g-16) .. (g >= 16), and the same plus DH.  A 16-lane row holds one token set's q or k,
        // both halves, so the q / k norm's sum over the head is one row sum.
        const int th = lane >> 5, g = lane & 31;
        const bool isq = g < 16;
        const int mc = 4 * (g & 15);         // channel within q or k (first half)
        const int lc = (isq ? 0 : D) + mc;   // q | k channel (first half)
        float *M = isq ? Q : K;
        float *img = isq ? qdst : qdst + C * D;
        const int t0w = 16 * wave + 8 * th;  // the lane's first token
        f4 wqk[2][4];
#pragma unroll
        for (int hp = 0; hp < 2; ++hp)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                wqk[hp][j] = *reinterpret_cast<const f4 *>(a.conv_w + (size_t)gchan(lc + DH * hp + j) * 4);
        raw4 rw[2][11];
#pragma unroll
        for (int hp = 0; hp < 2; ++hp)
#pragma unroll
            for (int i = 0; i < 11; ++i) rw[hp][i] = ld_raw(min(max(t0w - 3 + i, tmin), Lc - 1), lc + DH * hp);
        const bool head_rows = c == 0 && t0w == 0;  // the first three rows precede the call
        f4 hs[2][3] = {};
        if (head_rows)
#pragma unroll
            for (int hp = 0; hp < 2; ++hp)
#pragma unroll
                for (int i = 0; i < 3; ++i) hs[hp][i] = hist4(i - 3, lc + DH * hp);
        f4 y[2][8];
#pragma unroll
        for (int hp = 0; hp < 2; ++hp) {
            f4 xs[11];
#pragma unroll
            for (int i = 0; i < 11; ++i) xs[i] = (i < 3 && head_rows) ? hs[hp][i < 3 ? i : 0] : cvt(rw[hp][i]);
#pragma unroll
            for (int tt = 0; tt < 8; ++tt) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    float v = conv4(wqk[hp][j], xs[tt][j], xs[tt + 1][j], xs[tt + 2][j], xs[tt + 3][j]);
                    if constexpr (QKN) v = v * sigmoid_f(v);
                    y[hp][tt][j] = t0w + tt < Lc ? v : 0.f;
                }
            }
        }
#pragma unroll
        for (int tt = 0; tt < 8; ++tt) {
            const int t = t0w + tt;
            if constexpr (QKN) {  // unit length (+1e-6) over the head's channels; q also / sqrt(d)
                float ss = 0.f;
#pragma unroll
                for (int hp = 0; hp < 2; ++hp)
#pragma unroll
                    for (int j = 0; j < 4; ++j) ss += y[hp][tt][j] * y[hp][tt][j];
                ss = row16_sum(ss);
                const float sc = rsqrt_f(ss + 1e-6f) * (isq ? 1.0f / sqrtf((float)D) : 1.0f);
#pragma unroll
                for (int hp = 0; hp < 2; ++hp)
#pragma unroll
                    for (int j = 0; j < 4; ++j) y[hp][tt][j] *= sc;
            }
            MH::put4(M, t, mc, y[0][tt]);
            MQ::put4(img, t, mc, y[0][tt]);
            MQ::put4(img, t, mc + DH, y[1][tt]);
        }
        asm volatile("" : "+v"(gin.al), "+v"(gin.be), "+v"(gin.alog), "+v"(gin.dtb));  // loaded by now
        if (wave < min(R, L::heads)) gate_put(wave, gin);
        lds_barrier();  // the first half of q and k and the first heads' gates are in LDS
        gram();
        lds_barrier();  // every wave has read the first half
#pragma unroll
        for (int tt = 0; tt < 8; ++tt) MH::put4(M, t0w + tt, mc, y[1][tt]);
        lds_barrier();  // the second half is in LDS
        gram();
    }
    lds_barrier();  // q and k are consumed: their space holds A / T and P from here on
#pragma unroll 1
    for (int hh = 0; hh < R; ++hh) {
        const int h = hk * R + hh;
        if (hh > 0) lds_barrier();  // the previous head's T, P and gates are written out
        if (hh > 0 && hh % L::heads == 0) {  // the next group of heads' gates
            if (wave < min(R - hh, L::heads)) gate_put(hh + wave, gate_load(hh + wave));
            lds_barrier();
        }
        const double *Gam = reinterpret_cast<const double *>(gate_slot(hh));
        const float *gam = gate_slot(hh) + 2 * C, *bet = gam + C, *dec = bet + C;
        {
            float *Dm = wave < 2 ? Tm : Pm;
            // Every gate this lane's 20 entries use is read before any entry is formed, and the
            // entries are selected, not branched to: a read under a lane condition would cost an
            // LDS round trip per entry.
            double gt[5][4], gs[5];
            float bt[5][4];
#pragma unroll
            for (int jt = 0; jt < 5; ++jt) {
                gs[jt] = Gam[16 * tile_ct(jt) + (lane & 15)];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 16 * tile_rt(jt) + (lane >> 4) * 4 + r;
                    gt[jt][r] = Gam[t];
                    bt[jt][r] = bet[t];
                }
            }
#pragma unroll
            for (int jt = 0; jt < 5; ++jt) {
                const int rt = tile_rt(jt), ct = tile_ct(jt);
                const int s_ = 16 * ct + (lane & 15);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 16 * rt + (lane >> 4) * 4 + r;
                    const float ratio = exp_decay((float)(gt[jt][r] - gs[jt]));
                    const float av = s_ < t ? bt[jt][r] * ratio * tiles[jt][r] : 0.f;
                    const float pv = s_ <= t ? ratio * tiles[jt][r] : 0.f;
                    Dm[t * kCP + s_] = wave < 2 ? av : pv;
                }
            }
            // the six 16 x 16 blocks above the diagonal are zero
            for (int i = tid; i < 6 * 256; i += kPThreads) {
                const int bk = i >> 8, e = i & 255;
                const int rt = bk < 3 ? 0 : (bk < 5 ? 1 : 2), ct = bk < 3 ? bk + 1 : (bk < 5 ? bk - 1 : 3);
                const int at = (16 * rt + (e >> 4)) * kCP + 16 * ct + (e & 15);
                Tm[at] = 0.f;
                Pm[at] = 0.f;
            }
        }
        lds_barrier();
        // ---- T = (I + A)^-1: 16x16 diagonal blocks by forward substitution (wave w, lane c < 16
        // solves column c of block w), then the blocks below them
        if (lane < 16) {
            const int wv = wave, cc = lane;
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float acc = (r == cc) ? 1.f : 0.f;
#pragma unroll
                for (int s_ = 0; s_ < r; ++s_) acc -= Tm[(16 * wv + r) * kCP + 16 * wv + s_] * x[s_];
                x[r] = (r < cc) ? 0.f : acc;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) Tm[(16 * wv + r) * kCP + 16 * wv + cc] = x[r];
        }
        lds_barrier();
        // T_10 = -T_11 A_10 T_00 (wave 0) and T_32 = -T_33 A_32 T_22 (wave 1), the product A T
        // parked in the scratch; T_ij = -T_ii (sum_k A_ik T_kj) for the 32 x 32 block below
        float *scr_all = reinterpret_cast<float *>(smem + L::scr);
        float *scr = scr_all + wave * 256;  // [16][16] per wave
        auto park = [&](f4 v) {
#pragma unroll
            for (int r = 0; r < 4; ++r) scr[((lane >> 4) * 4 + r) * 16 + (lane & 15)] = v[r];
        };
        auto blk16s = [&](const float *X, int xr0, int xc0, const float *Y, f4 acc) {  // acc += X(block) Y
#pragma unroll
            for (int st2 = 0; st2 < 4; ++st2) {
                const int kk = 4 * st2 + (lane >> 4);
                acc = mfma4f32(X[(xr0 + (lane & 15)) * kCP + xc0 + kk], Y[kk * 16 + (lane & 15)], acc);
            }
            return acc;
        };
        auto put_neg = [&](int r0, int c0, f4 v) {
#pragma unroll
            for (int r = 0; r < 4; ++r) Tm[(r0 + (lane >> 4) * 4 + r) * kCP + c0 + (lane & 15)] = -v[r];
        };
        if (wave < 2) {
            const int i = wave == 0 ? 1 : 3, j = i - 1;
            park(blk16(Tm, 16 * i, 16 * j, Tm, 16 * j, 16 * j, f4{0.f, 0.f, 0.f, 0.f}, lane));
            put_neg(16 * i, 16 * j, blk16s(Tm, 16 * i, 16 * i, scr, f4{0.f, 0.f, 0.f, 0.f}));
        }
        lds_barrier();
        const int r3 = 2 + (wave >> 1), c3 = wave & 1;  // block (r3, c3) of the lower-left 32 x 32
        {  // X_rc = A_r0 T_0c + A_r1 T_1c
            f4 x = blk16(Tm, 16 * r3, 16, Tm, 16, 16 * c3, f4{0.f, 0.f, 0.f, 0.f}, lane);
            if (c3 == 0) x = blk16(Tm, 16 * r3, 0, Tm, 0, 0, x, lane);
            park(x);
        }
        lds_barrier();
        {  // T_2c = -T_22 X_2c ;  T_3c = -(T_32 X_2c + T_33 X_3c)  (X_2c parked by wave c, X_3c by wave 2 + c)
            f4 acc = blk16s(Tm, 16 * r3, 32, scr_all + c3 * 256, f4{0.f, 0.f, 0.f, 0.f});
            if (r3 == 3) acc = blk16s(Tm, 48, 48, scr, acc);
            put_neg(16 * r3, 16 * c3, acc);
        }
        lds_barrier();

        // ---- T, P and the gates for the scan (T and P as Tri images)
        {
            using MT = Tri<F32>;
            static_assert(MT::floats == kTriFloats, "the workspace holds Tri images");
            const size_t ch = (size_t)c * a.n_vh + h;
            float *tdst = a.ws + w.t + ch * kTriFloats;
            float *pdst = a.ws + w.p + ch * kTriFloats;
            for (int g = tid; g < C * C / 8; g += kPThreads) {
                const int r = g / (C / 8), c0 = (g % (C / 8)) * 8;
                float x[8];
                load8(Tm + r * kCP + c0, x);
                MT::put8(tdst, r, c0, x);
                load8(Pm + r * kCP + c0, x);
                MT::put8(pdst, r, c0, x);
            }
            if (tid < C) {
                float *g = a.ws + w.g + ch * kGateRec;
                g[tid] = gam[tid];
                g[C + tid] = bet[tid];
                g[2 * C + tid] = dec[tid];
                g[3 * C + tid] = 0.f;
            }
        }
    }
}

// ============================== kernel 2: the chunk chain ==============================
// Per chunk, for this workgroup's kSR value rows (S block kSR x d, rows i, key columns j):
//   A: Y^T = beta (V^T - (S K^T) diag(gamma))     V convolved here from the raw activations
//   B: U^T = Y^T T^T
//   C: O   = diag(gamma) Q S^T + P U ;  S' = gamma_C S + U^T diag(dec) K
// Compute wave w owns tokens 16 w .. 16 w + 15 of A, B and the readout, for every 16-row tile of the
// block, so every q, k, T and P element is read from LDS once per chunk; its S' share is key
// columns 16 (2 w) .. 16 (2 w) + 31 (d = 128).  Each wave reads the whole S block into registers as
// MFMA operand fragments at the start of a chunk and uses it in A for both products that need it,
// K S^T and Q S^T (the latter kept until C); it holds its own S' tiles in fp32.  Four producer waves
// move the next operands in with global_load_lds while the compute waves work: q and k of c + 1 once
// A has read them (the key columns C needs are held in registers from A on), T, P, v and the gates
// of c + 1 once B is done; every transfer of c + 1 is waited for before the chunk starts.
constexpr int kScanCompute = kChunk / 16;  // compute waves: one 16-token tile each
constexpr int kProducers = 4;
constexpr int kScanThreads = 64 * (kScanCompute + kProducers);

// s_waitcnt immediate: wait until at most n vector-memory operations are outstanding (gfx9
// encoding: vmcnt bits 3:0 and 15:14; expcnt and lgkmcnt left at their maxima).
constexpr int vmcnt_imm(int n) { return 0x0F70 | (n & 0xF) | ((n >> 4) << 14); }

template <int D, bool ACT_BF16, bool QKN>
__global__ __launch_bounds__(kScanThreads) void prefill_scan_kernel(PrefillArgs a)
{
    constexpr bool F32 = !ACT_BF16;
    using L = ScanLds<D, ACT_BF16>;
    constexpr int C = kChunk;
    constexpr int NB = D / kSR;   // row blocks per value head
    constexpr int KK = D / 32;    // 32-deep steps over the key dimension
    using MK = Mat<F32, C, D>;    // q and k images
    using MT = Tri<F32>;          // T and P images
    using MS = Mat<F32, kSR, D>;  // S block
    using MY = Mat<F32, kSR, C>;  // Y^T
    constexpr int SCT = D / 16 / kScanCompute;     // S' column tiles per compute wave
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const bool producer = wave >= kScanCompute;
    const int R = a.n_vh / a.n_kh;
    // workgroups are dealt to the 8 XCDs in turn: keep the row blocks of a key head's value heads on
    // one XCD, so the operand images they all read are fetched into that XCD's L2 once
    const int nwg = a.n_vh * NB;
    const int idx = nwg % 8 == 0 ? (blockIdx.x % 8) * (nwg / 8) + blockIdx.x / 8 : blockIdx.x;
    const int h = idx / NB, blk = idx % NB;
    const int hk = h / R;
    const int T = a.T;
    const int Cc = a.C;
    const int nchunks = (T + C - 1) / C;
    const PrefillWs w = prefill_ws(D, a.n_kh, a.n_vh, T);
    const int li = lane & 15, lg = lane >> 4;  // fragment row / column, 8-wide k group
    const int vch0 = 2 * a.n_kh * D + h * D + blk * kSR;  // the block's first v channel

    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    float *Kc = reinterpret_cast<float *>(smem + L::kb);
    float *Q = reinterpret_cast<float *>(smem + L::q);
    float *Tm = reinterpret_cast<float *>(smem + L::tm);
    float *Pb = reinterpret_cast<float *>(smem + L::pm);
    unsigned char *Vr = smem + L::vb;
    float *Gb = reinterpret_cast<float *>(smem + L::gb);
    float *Yp = reinterpret_cast<float *>(smem + L::yp);
    float *Up = reinterpret_cast<float *>(smem + L::up);  // U^T, operand form
    float *Sx = reinterpret_cast<float *>(smem + L::sx);

    // ---- the producers' transfers (lane i of a global_load_lds lands at the base + 16 i).  N16
    // 16-byte pieces, a multiple of 64 per producer wave: a fixed number of whole-wave transfers per
    // wave, unrolled, each at a wave-uniform LDS base.
    const int pw = __builtin_amdgcn_readfirstlane(wave - kScanCompute);  // producer index
    auto dma = [&](auto n16_c, const float *g, float *l) {
        constexpr int N16 = decltype(n16_c)::value;
        static_assert(N16 % (64 * kProducers) == 0, "whole-wave transfers, the same count on every producer");
#pragma unroll
        for (int k = 0; k < N16 / (64 * kProducers); ++k) {
            const int i0 = 64 * (pw + k * kProducers);
            lds_dma16(g + 4 * (i0 + lane), l + 4 * i0);
        }
    };
    auto qk_img = [&](int cc, int which) { return a.ws + w.qk + (((size_t)cc * a.n_kh + hk) * 2 + which) * C * D; };
    auto chunk_rec = [&](int cc) { return (size_t)cc * a.n_vh + h; };
    using img16 = std::integral_constant<int, C * D / 4>;  // a q or k image in 16-byte pieces
    using half16 = std::integral_constant<int, C * D / 8>;
    using tri16 = std::integral_constant<int, kTriFloats / 4>;  // a T or P image
    auto issue_k = [&](int cc, int half) {  // one half of the k image
        dma(half16{}, qk_img(cc, 1) + half * (C * D / 2), Kc + half * (C * D / 2));
    };
    auto issue_q = [&](int cc) { dma(img16{}, qk_img(cc, 0), Q + (cc & 1) * C * D); };
    auto issue_t = [&](int cc) { dma(tri16{}, a.ws + w.t + chunk_rec(cc) * kTriFloats, Tm); };
    auto issue_pg = [&](int cc) {  // P and the gate record of chunk cc (one transfer per producer each)
        dma(tri16{}, a.ws + w.p + chunk_rec(cc) * kTriFloats, Pb + (cc & 1) * kTriFloats);
        if (lane < kGateRec / 4 / kProducers) {
            const int i0 = pw * (kGateRec / 4 / kProducers);
            lds_dma16(a.ws + w.g + chunk_rec(cc) * kGateRec + 4 * (i0 + lane), Gb + (cc & 1) * kGateRec + 4 * i0);
        }
    };
    auto issue_v = [&](int cc) {  // raw v rows of chunk cc
        constexpr int lpr = L::vrow / 16;  // lanes per raw row
#pragma unroll
        for (int k = 0; k < (L::vdmas + kProducers - 1) / kProducers; ++k) {
            const int j = pw + k * kProducers;
            if (j < L::vdmas) {
                const int row = j * L::vrows_per_dma + lane / lpr;
                const int tok = min(max(cc * C - 3 + row, 0), T - 1);  // rows outside the call are never used
                const unsigned char *g = static_cast<const unsigned char *>(a.qkv) +
                                         ((size_t)tok * Cc + vch0) * (ACT_BF16 ? 2 : 4) + 16 * (lane % lpr);
                lds_dma16(g, Vr + 1024 * j);
            }
        }
    };
    // L2 touch of chunk cc's operands, a chunk before their transfers into LDS: one dword of every
    // 128-byte line of this workgroup's share of the key head's q and k images and of the value
    // head's T and P (one 4-byte transfer per producer wave, 16 lines each; slots past the share
    // repeat its first line).  It only warms the cache: what lands in LDS is never read.
    auto issue_touch = [&](int cc) {
        constexpr int qk_lines = 2 * C * D * 4 / 128, tp_lines = kTriFloats * 4 / 128;
        const int grp = R * NB, j = (h % R) * NB + blk;  // workgroups of the key head, this one's index
        const int nq = (qk_lines + grp - 1) / grp, ntp = (tp_lines + NB - 1) / NB;
        const int sl = 16 * pw + (lane & 15);
        const int in_t = sl - nq, in_p = sl - nq - ntp;
        const float *src = in_p >= 0 && in_p < ntp ? a.ws + w.p + chunk_rec(cc) * kTriFloats + 32 * min(blk * ntp + in_p, tp_lines - 1)
                         : in_t >= 0 && in_t < ntp ? a.ws + w.t + chunk_rec(cc) * kTriFloats + 32 * min(blk * ntp + in_t, tp_lines - 1)
                                                   : qk_img(cc, 0) + 32 * min(sl < nq ? j * nq + sl : j * nq, qk_lines - 1);
        lds_dma4(src, smem + L::touch);
    };
    // transfers per producer wave: T or P, a q image (uniform), and one gate transfer each
    constexpr int NT = kTriFloats / 4 / (64 * kProducers);
    constexpr int NQ = C * D / 4 / (64 * kProducers);
    static_assert(NT * 64 * kProducers == kTriFloats / 4 && NT + NQ + 1 < 64, "T and P split evenly over the producers");
    static_assert(kGateRec / 4 / kProducers <= 64, "a gate record is one partial transfer per producer");

    // The producers and the compute waves run separate loops with the same three barriers per
    // chunk.  (In one shared loop the compiler would have to assume a transfer into LDS in flight
    // on the compute waves' path too, and make them wait for all their own vector-memory operations
    // before touching LDS.)
    // A buffer is refilled as soon as the phase that reads it is done, and the transfers of c + 1
    // are spread over the three phases of c in proportion to their length, so that no producer
    // reaches a barrier after the compute waves: P, the gates and q (double buffered) during A;
    // half of k and v during B (A has read k and v of c); the other half of k and T during C.  T is
    // issued last and needed only by B, so the chunk start waits for everything else and the
    // barrier after A for T.  The operands of c + 2 are touched into L2 during A of c, so the
    // transfers of c + 1 that start late in c find them there rather than in HBM.
    if (producer) {
        issue_pg(0);
        issue_q(0);
        issue_k(0, 0);
        issue_v(0);
        issue_k(0, 1);
        issue_touch(min(1, nchunks - 1));
        issue_t(0);
#pragma unroll 1
        for (int c = 0; c < nchunks; ++c) {
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(NT));  // q, k, v, P, gates of c have landed (T may travel)
            lds_barrier();                                // chunk start
            if (c + 1 < nchunks) {
                issue_pg(c + 1);
                issue_q(c + 1);
                issue_touch(min(c + 2, nchunks - 1));
                __builtin_amdgcn_s_waitcnt(vmcnt_imm(NT + 1 + NQ + 1));  // T of c (P, gates, q of c + 1, the touch may travel)
            } else {
                __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
            }
            lds_barrier();  // A done: q, k and v of c are consumed; T of c has landed
            if (c + 1 < nchunks) {
                issue_k(c + 1, 0);
                issue_v(c + 1);
            }
            lds_barrier();  // B done: T of c is consumed
            if (c + 1 < nchunks) {
                issue_k(c + 1, 1);
                issue_t(c + 1);
            }
        }
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // no transfer into LDS outlives the workgroup
        return;
    }

    // ---- compute waves.  State: the S block's fp32 elements this wave produces (row 16 rt + li, key
    // columns 16 (SCT w + q2) + 4 lg .. + 3: S' is computed transposed, so a lane holds four
    // consecutive columns of one row), the conv taps and the conv-state rows of its v channels
    float *st = a.state + ((size_t)a.slot * a.n_vh + h) * D * D + (size_t)blk * kSR * D;
    float *Dp = reinterpret_cast<float *>(smem + L::dp);
    constexpr int RT = kRT;
    f4 sreg[RT][SCT];
    f4 wv[RT];
    float hist[RT][3];
    auto s_at = [&](int rt, int q2) { return (size_t)(16 * rt + li) * D + 16 * (SCT * wave + q2) + 4 * lg; };
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
        for (int q2 = 0; q2 < SCT; ++q2) sreg[rt][q2] = *reinterpret_cast<const f4 *>(st + s_at(rt, q2));
        const int vc = vch0 + 16 * rt + li;
        wv[rt] = *reinterpret_cast<const f4 *>(a.conv_w + (size_t)vc * 4);
#pragma unroll
        for (int m = 0; m < 3; ++m) hist[rt][m] = a.conv_state[((size_t)a.slot * 3 + m) * Cc + vc];
    }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int q2 = 0; q2 < SCT; ++q2) MS::put4(Sx, 16 * rt + li, 16 * (SCT * wave + q2) + 4 * lg, sreg[rt][q2]);
    auto raw_v = [&](int row, int ch) -> float {  // window row of the chunk, block channel
        if constexpr (ACT_BF16)
            return bf16_to_f32(reinterpret_cast<const uint16_t *>(Vr)[row * kSR + ch]);
        else
            return reinterpret_cast<const float *>(Vr)[row * kSR + ch];
    };
    const int t4 = 16 * wave + 4 * lg;  // this lane's four tokens in A and B
    const int tr = 16 * wave + li;      // this lane's token in the readout (computed transposed)

#pragma unroll 1
    for (int c = 0; c < nchunks; ++c) {
        const float *gam = Gb + (c & 1) * kGateRec;
        const float *bet = gam + C;
        const float *dec = bet + C;
        const float *Pm = Pb + (c & 1) * kTriFloats;
        const float *Qc = Q + (c & 1) * C * D;
        lds_barrier();  // chunk start: the operands of c and S are in LDS
        // ---- A: (K S^T)[t][i] for tokens t4 + r, rows 16 rt + li, and the readout's S Q^T [i][t]
        // for rows 16 rt + 4 lg + r, token tr; then Y^T[i][t] = beta_t (v_t[i] - gamma_t (K S^T)[t][i])
        Frag<F32> kf[SCT][2];  // K columns of this wave's S' tiles (C's A operand)
        f4 acc4[2 * RT] = {};  // K S^T of the row tiles, then S Q^T of the row tiles
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            const Frag<F32> kr = MK::load(Kc, tr, 32 * kk + 8 * lg);
            const Frag<F32> qr = MK::load(Qc, tr, 32 * kk + 8 * lg);
            Frag<F32> fa[2 * RT], fb[2 * RT];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const Frag<F32> sf = MS::load(Sx, 16 * rt + li, 32 * kk + 8 * lg);
                fa[rt] = kr;
                fb[rt] = sf;
                fa[RT + rt] = sf;
                fb[RT + rt] = qr;
            }
            mma_n<F32, 2 * RT>(fa, fb, acc4);
        }
#pragma unroll
        for (int q2 = 0; q2 < SCT; ++q2) {
            const int j0 = 16 * (SCT * wave + q2);
#pragma unroll
            for (int kk2 = 0; kk2 < 2; ++kk2) {
                if constexpr (F32) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) MK::get(Kc, 32 * kk2 + 8 * lg + e, j0 + li, kf[q2][kk2], e);
                } else {
                    kf[q2][kk2] = MK::load_col(Kc, 32 * kk2 + 8 * lg, j0, li);
                }
            }
        }
        {
            const f4 g4 = *reinterpret_cast<const f4 *>(gam + t4);
            const f4 b4 = *reinterpret_cast<const f4 *>(bet + t4);
            const bool from_state = c == 0 && t4 == 0;  // window rows 0..2 precede the call
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const int ch = 16 * rt + li;
                float xr[7];  // window rows t4 .. t4 + 6 of channel ch, every read issued before any use
#pragma unroll
                for (int m = 0; m < 7; ++m) xr[m] = raw_v(t4 + m, ch);
#pragma unroll
                for (int m = 0; m < 3; ++m) xr[m] = from_state ? hist[rt][m] : xr[m];
                f4 y;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float v = conv4(wv[rt], xr[r], xr[r + 1], xr[r + 2], xr[r + 3]);
                    if constexpr (QKN) v = v * sigmoid_f(v);
                    y[r] = b4[r] * (v - g4[r] * acc4[rt][r]);
                }
                MY::put4(Yp, ch, t4, y);
            }
        }
        lds_barrier();  // Y^T is in LDS; q, k and the raw v rows are consumed
        // ---- B: U[t][i] = sum_s T[t][s] Y[s][i]; U^T (and U^T diag(dec)) into LDS in operand form
        {
            f4 part[2 * RT] = {};  // the row tiles over tokens 0..31, then over 32..63
            // tokens 0..31 (waves 0, 1) have no T entries in columns 32..63
            const Frag<F32> t0 = MT::load(Tm, tr, 8 * lg), t1 = wave >= 2 ? MT::load(Tm, tr, 32 + 8 * lg) : Frag<F32>{};
            Frag<F32> fa[2 * RT], fb[2 * RT];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                fa[rt] = t0;
                fa[RT + rt] = t1;
                fb[rt] = MY::load(Yp, 16 * rt + li, 8 * lg);
                fb[RT + rt] = MY::load(Yp, 16 * rt + li, 32 + 8 * lg);
            }
            mma_n<F32, 2 * RT>(fa, fb, part);
            const f4 d4 = *reinterpret_cast<const f4 *>(dec + t4);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const f4 u = part[rt] + part[RT + rt];
                MY::put4(Up, 16 * rt + li, t4, u);
                if constexpr (!F32) MY::put4(Dp, 16 * rt + li, t4, u * d4);
            }
        }
        lds_barrier();  // U^T is in LDS; T is consumed
        // ---- C: O^T = (S Q^T) diag(gamma) + U^T P^T, then S'^T = gamma_C S^T + K^T (U^T diag(dec))^T.
        // S' goes into LDS for every wave; no wave reads S there before the next chunk.
        {
            const float gC = gam[C - 1];
            const float gt = gam[tr];
            Frag<F32> uf[RT][2], udf[RT][2], pr[2];  // [tile][token half], [token half]
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                pr[h2] = h2 == 0 || wave >= 2 ? MT::load(Pm, tr, 32 * h2 + 8 * lg) : Frag<F32>{};
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
                    uf[rt][h2] = MY::load(Up, 16 * rt + li, 32 * h2 + 8 * lg);
                    if constexpr (F32) {
#pragma unroll
                        for (int e = 0; e < 8; ++e) udf[rt][h2].v[e] = uf[rt][h2].v[e] * dec[32 * h2 + 8 * lg + e];
                    } else {
                        udf[rt][h2] = MY::load(Dp, 16 * rt + li, 32 * h2 + 8 * lg);
                    }
                }
            }
            // accumulators: the readout of the row tiles, then S'^T of (row tile, column tile)
            constexpr int NA = RT + RT * SCT;
            f4 acc6[NA];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) acc6[rt] = acc4[RT + rt] * gt;
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int q2 = 0; q2 < SCT; ++q2) acc6[RT + rt * SCT + q2] = sreg[rt][q2] * gC;
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                Frag<F32> fa[NA], fb[NA];
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
                    fa[rt] = uf[rt][h2];
                    fb[rt] = pr[h2];
                }
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                    for (int q2 = 0; q2 < SCT; ++q2) {
                        fa[RT + rt * SCT + q2] = kf[q2][h2];
                        fb[RT + rt * SCT + q2] = udf[rt][h2];
                    }
                mma_n<F32, NA>(fa, fb, acc6);
            }
            // the readout: rows 16 rt + 4 lg .. + 3 of token tr, four consecutive floats (whole
            // chunks fit the readout)
            float *orow = a.ws + w.o + ((size_t)(c * C + tr) * a.n_vh + h) * D + blk * kSR + 4 * lg;
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) *reinterpret_cast<f4 *>(orow + 16 * rt) = acc6[rt];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int q2 = 0; q2 < SCT; ++q2) {
                    sreg[rt][q2] = acc6[RT + rt * SCT + q2];
                    MS::put4(Sx, 16 * rt + li, 16 * (SCT * wave + q2) + 4 * lg, sreg[rt][q2]);
                }
        }
    }
    // ---- the state block after the last token
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int q2 = 0; q2 < SCT; ++q2) *reinterpret_cast<f4 *>(st + s_at(rt, q2)) = sreg[rt][q2];
}

// N consecutive activations (bf16 or fp32) at element offset off, as fp32; off is a multiple of N.
template <bool BF16, int N>
__device__ __forceinline__ void load_n(const void *p, size_t off, float (&x)[N])
{
    if constexpr (BF16) {
        const uint16_t *q = static_cast<const uint16_t *>(p) + off;
#pragma unroll
        for (int e = 0; e < N; e += 4) {
            const uint2 u = *reinterpret_cast<const uint2 *>(q + e);
            x[e] = bf16_to_f32((uint16_t)(u.x & 0xffffu));
            x[e + 1] = bf16_to_f32((uint16_t)(u.x >> 16));
            x[e + 2] = bf16_to_f32((uint16_t)(u.y & 0xffffu));
            x[e + 3] = bf16_to_f32((uint16_t)(u.y >> 16));
        }
    } else {
        const float *q = static_cast<const float *>(p) + off;
#pragma unroll
        for (int e = 0; e < N; e += 4) {
            const f4 v = *reinterpret_cast<const f4 *>(q + e);
            x[e] = v[0];
            x[e + 1] = v[1];
            x[e + 2] = v[2];
            x[e + 3] = v[3];
        }
    }
}

// load_n with non-temporal loads, for data read once (the norm kernel's readout and z: 1.5 us of
// the prefill's 397 at 8192 tokens)
template <bool BF16, int N>
__device__ __forceinline__ void load_n_nt(const void *p, size_t off, float (&x)[N])
{
    typedef unsigned int u2v __attribute__((ext_vector_type(2)));
    if constexpr (BF16) {
        const uint16_t *q = static_cast<const uint16_t *>(p) + off;
#pragma unroll
        for (int e = 0; e < N; e += 4) {
            const u2v u = __builtin_nontemporal_load(reinterpret_cast<const u2v *>(q + e));
            x[e] = bf16_to_f32((uint16_t)(u.x & 0xffffu));
            x[e + 1] = bf16_to_f32((uint16_t)(u.x >> 16));
            x[e + 2] = bf16_to_f32((uint16_t)(u.y & 0xffffu));
            x[e + 3] = bf16_to_f32((uint16_t)(u.y >> 16));
        }
    } else {
        const float *q = static_cast<const float *>(p) + off;
#pragma unroll
        for (int e = 0; e < N; e += 4) {
            const f4 v = __builtin_nontemporal_load(reinterpret_cast<const f4 *>(q + e));
            x[e] = v[0];
            x[e + 1] = v[1];
            x[e + 2] = v[2];
            x[e + 3] = v[3];
        }
    }
}

template <bool BF16, int N>
__device__ __forceinline__ void store_n(void *p, size_t off, const float (&y)[N])
{
    if constexpr (BF16) {
        uint16_t *q = static_cast<uint16_t *>(p) + off;
#pragma unroll
        for (int e = 0; e < N; e += 4)
            *reinterpret_cast<uint2 *>(q + e) = uint2{(uint32_t)f32_to_bf16(y[e]) | ((uint32_t)f32_to_bf16(y[e + 1]) << 16),
                                                      (uint32_t)f32_to_bf16(y[e + 2]) | ((uint32_t)f32_to_bf16(y[e + 3]) << 16)};
    } else {
        float *q = static_cast<float *>(p) + off;
#pragma unroll
        for (int e = 0; e < N; e += 4) *reinterpret_cast<f4 *>(q + e) = f4{y[e], y[e + 1], y[e + 2], y[e + 3]};
    }
}

// out = o / sqrt(mean(o^2) + eps) * norm_w * silu(z) per (token, head): 16 lanes per row, each
// 16-lane group takes kNormRows rows 16 apart and issues all their loads before any arithmetic.
// The blocks after the rows write the conv state after the last token.
constexpr int kNormRows = 4;

template <int D, bool ACT_BF16, bool OUT_BF16>
__global__ __launch_bounds__(256) void prefill_norm_kernel(PrefillArgs a)
{
    constexpr int EPL = D / 16;
    const int grp = threadIdx.x >> 4, cg = threadIdx.x & 15;
    const int nrows = a.T * a.n_vh;
    const int row_blocks = (nrows + 16 * kNormRows - 1) / (16 * kNormRows);
    if ((int)blockIdx.x < row_blocks) {
        const int row0 = blockIdx.x * 16 * kNormRows + grp;
        float ov[kNormRows][EPL], zv[kNormRows][EPL];
#pragma unroll
        for (int k = 0; k < kNormRows; ++k) {
            const int row = row0 + 16 * k;
            if (row < nrows) {  // the same for the 16 lanes of a row
                const size_t base = (size_t)row * D + cg * EPL;
                load_n_nt<false, EPL>(a.ws, base, ov[k]);  // the readout sits at the start of the workspace
                load_n_nt<ACT_BF16, EPL>(a.z, base, zv[k]);
            }
        }
        float nw[EPL];
        load_n<false, EPL>(a.norm_w, cg * EPL, nw);
#pragma unroll
        for (int k = 0; k < kNormRows; ++k) {
            const int row = row0 + 16 * k;
            if (row < nrows) {
                float ss = 0.f;
#pragma unroll
                for (int e = 0; e < EPL; ++e) ss += ov[k][e] * ov[k][e];
                ss = row16_sum(ss);
                const float inv = 1.0f / sqrtf(ss / (float)D + a.eps);
                float y[EPL];
#pragma unroll
                for (int e = 0; e < EPL; ++e) {
                    const float zz = zv[k][e];
                    y[e] = ov[k][e] * inv * nw[e] * (zz * sigmoid_f(zz));
                }
                store_n<OUT_BF16, EPL>(a.out, (size_t)row * D + cg * EPL, y);
            }
        }
    } else {
        // conv state after the last token = the last three rows of concat(old conv state, qkv);
        // one thread per channel
        const int gc = (blockIdx.x - row_blocks) * 256 + threadIdx.x;
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

size_t prefill_workspace_bytes(int d, int n_kh, int n_vh, int T)
{
    return sizeof(float) * prefill_ws(d, n_kh, n_vh, T).total;
}

size_t prefill_lds_bytes(int d, bool act_bf16)
{
    const size_t prep = d == 128 ? PrepLds<128>::total : PrepLds<64>::total;
    const size_t scan = d == 128 ? (act_bf16 ? ScanLds<128, true>::total : ScanLds<128, false>::total)
                                 : (act_bf16 ? ScanLds<64, true>::total : ScanLds<64, false>::total);
    return prep > scan ? prep : scan;
}

template <int D, bool AB, bool OB, bool QKN>
static hipError_t launch_prefill_t(const PrefillArgs &a, hipStream_t stream)
{
    const int nchunks = (a.T + kChunk - 1) / kChunk;
    const size_t prep_lds = PrepLds<D>::total;
    hipLaunchKernelGGL((prefill_prep_kernel<D, AB, QKN>), dim3(nchunks * a.n_kh), dim3(kPThreads), prep_lds, stream, a);
    if (hipError_t e = hipGetLastError()) return e;
    hipLaunchKernelGGL((prefill_scan_kernel<D, AB, QKN>), dim3(a.n_vh * (D / kSR)), dim3(kScanThreads),
                       (ScanLds<D, AB>::total), stream, a);
    if (hipError_t e = hipGetLastError()) return e;
    const long rows = (long)a.T * a.n_vh;
    const long row_blocks = (rows + 16 * kNormRows - 1) / (16 * kNormRows);
    const long conv_blocks = (a.C + 255) / 256;
    hipLaunchKernelGGL((prefill_norm_kernel<D, AB, OB>), dim3((unsigned)(row_blocks + conv_blocks)), dim3(256), 0, stream,
                       a);
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
