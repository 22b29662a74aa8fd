// gdn_verify.hip - fused chain verify for the Gated DeltaNet speculative-decode step (gfx950).
//
// One workgroup per (batch entry, key head) handles every value head that reads that key head
// (H_v / H_k of them), so each q / k conv channel and each conv_state element has exactly one
// owner: the conv window can be read and then advanced in place without a second pass.
//
// The fp32 recurrent state S (d_v x d_k per value head) stays in VGPRs across all tokens and
// is read and written once from HBM.  Lane layout of one value head (NW waves):
//   lane = 16 * rg + cg,  rg in [0,4) picks a row group, cg in [0,16) a column group
//   rows  of register i : wave_in_head * 4*RPL + 4*i + rg          (RPL rows per lane)
//   cols  of chunk c4   : 64*c4 + 4*cg + e,  e in [0,4)             (CPL = d/16 columns)
// so one float4 store instruction covers 4 consecutive rows x 64 contiguous columns: every
// 128-byte line of the per-token capture is written whole by a single instruction.  Both
// contractions over the key index (S k and S q) finish with a 16-lane DPP sum.
//
// Per token (Yang, Kautz & Hatamizadeh 2024, gated delta rule):
//   p = S k,  u = beta (v - rho p),  S <- rho S + u k^T,  o = rho (S_old q) + (k.q) u  (= S_new q)
// The capture of S after every token (lucebox-hub internal.h, struct TargetCache,
// ssm_intermediate) is streamed out with nontemporal stores; the RMS norm + SiLU(z) epilogue
// (ssm_norm, z projection: internal.h, struct TargetLayer) runs per token tile from LDS.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

template <int D, int NW>
struct Geo {
    static constexpr int RPL = D / (NW * 4);  // state rows per lane
    static constexpr int CPL = D / 16;        // state columns per lane
    static constexpr int NC4 = CPL / 4;       // float4 column chunks per lane
    static constexpr int RPW = 4 * RPL;       // rows per wave
    static_assert(RPL >= 1 && NC4 >= 1, "bad geometry");
    // LDS position of natural row r in the per-lane-contiguous order used for v and o.
    __device__ static int perm(int r)
    {
        const int w = r / RPW, rem = r % RPW;
        return w * RPW + (rem & 3) * RPL + (rem >> 2);
    }
};

template <int D>
struct WavesPerHead;
template <>
struct WavesPerHead<128> {
    static constexpr int value = 4;
};
template <>
struct WavesPerHead<64> {
    static constexpr int value = 2;
};

__device__ __forceinline__ void store_nt(float *p, f4 v) { __builtin_nontemporal_store(v, reinterpret_cast<f4 *>(p)); }

template <int D, bool ACT_BF16, bool OUT_BF16, bool QKN, bool CAP>
__global__ __launch_bounds__(1024) void verify_chain_kernel(VerifyArgs a)
{
    constexpr int NW = WavesPerHead<D>::value;
    using G = Geo<D, NW>;
    constexpr int TT = kTokenTile;
    const int R = a.n_vh / a.n_kh;
    const int nthr = blockDim.x;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int nwaves = nthr >> 6;
    const int hl = wave / NW, wih = wave % NW;
    const int rg = lane >> 4, cg = lane & 15;

    const int b = blockIdx.x / a.n_kh;
    const int hk = blockIdx.x % a.n_kh;
    const int h = hk * R + hl;
    const int s = a.slot_ids[b];
    if (s < 0 || s >= a.n_pool) return;  // uniform over the workgroup

    extern __shared__ float smem[];
    float *ks = smem;                  // [TT][D]
    float *qs = ks + TT * D;           // [TT][D]
    float *vs = qs + TT * D;           // [R][TT][D]   rows in perm order
    float *os = vs + R * TT * D;       // [R][TT][D]   rows in perm order
    float *rb = os + R * TT * D;       // [R][TT][2]   (rho, beta)
    float *kqs = rb + R * TT * 2;      // [TT]         k . q

    const int C = a.C;
    const int T = a.T;
    const int nch = (2 + R) * D;
    const int q0 = hk * D, k0 = a.n_kh * D + hk * D, v0 = 2 * a.n_kh * D + hk * R * D;
    float *cs_s = a.conv_state + (size_t)s * 3 * C;
    const size_t hd = (size_t)D * D;

    // ---- state -> registers
    float S[G::RPL][G::CPL];  // S[i][4 c4 + e] = state row (row0 + 4 i), column (64 c4 + 4 cg + e)
    const int row0 = wih * G::RPW + rg;
    float *st_ptr = a.state + ((size_t)s * a.n_vh + h) * hd + (size_t)row0 * D + cg * 4;
#pragma unroll
    for (int i = 0; i < G::RPL; ++i)
#pragma unroll
        for (int c4 = 0; c4 < G::NC4; ++c4) {
            const f4 v = *reinterpret_cast<const f4 *>(st_ptr + (size_t)(4 * i) * D + 64 * c4);
#pragma unroll
            for (int e = 0; e < 4; ++e) S[i][4 * c4 + e] = v[e];
        }

    float *cap_ptr = nullptr;
    size_t cap_tstride = 0;
    if constexpr (CAP) {
        cap_ptr = a.cap_ssm + ((size_t)s * a.t_cap * a.n_vh + h) * hd + (size_t)row0 * D + cg * 4;
        cap_tstride = (size_t)a.n_vh * hd;
    }

    auto xext = [&](int r, int gc) -> float {
        return r < 3 ? cs_s[(size_t)r * C + gc]
                     : load_act<ACT_BF16>(a.qkv, ((size_t)b * T + (r - 3)) * C + gc);
    };

#pragma unroll 1
    for (int t0 = 0; t0 < T; t0 += TT) {
        const int nt = min(TT, T - t0);
        // ---- depthwise causal conv of this tile (one thread per channel)
#pragma unroll 1
        for (int lc = tid; lc < nch; lc += nthr) {
            int gc;
            float *dst;
            if (lc < D) {
                gc = q0 + lc;
                dst = qs + lc;
            } else if (lc < 2 * D) {
                gc = k0 + (lc - D);
                dst = ks + (lc - D);
            } else {
                const int vr = lc - 2 * D;
                gc = v0 + vr;
                dst = vs + (vr / D) * TT * D + G::perm(vr % D);
            }
            const f4 w = *reinterpret_cast<const f4 *>(a.conv_w + (size_t)gc * 4);
            float x0 = xext(t0, gc), x1 = xext(t0 + 1, gc), x2 = xext(t0 + 2, gc);
            float *cc = CAP ? a.cap_conv + (size_t)s * (3 + a.t_cap) * C + gc : nullptr;
            if (CAP && t0 == 0) {
                cc[0] = x0;
                cc[(size_t)C] = x1;
                cc[(size_t)2 * C] = x2;
            }
#pragma unroll 2
            for (int t = 0; t < nt; ++t) {
                const float x3 = xext(t0 + t + 3, gc);
                float y = w[0] * x0 + w[1] * x1 + w[2] * x2 + w[3] * x3;
                if constexpr (QKN) y = y * sigmoid_f(y);
                dst[t * D] = y;
                if constexpr (CAP) cc[(size_t)(t0 + t + 3) * C] = x3;
                x0 = x1;
                x1 = x2;
                x2 = x3;
            }
        }
        // ---- per-token gate and beta
        for (int i = tid; i < nt * R; i += nthr) {
            const int t = i / R, hh = i % R, h2 = hk * R + hh;
            const size_t tok = ((size_t)b * T + t0 + t) * a.n_vh + h2;
            const float al = load_act<ACT_BF16>(a.alpha, tok);
            const float be = load_act<ACT_BF16>(a.beta, tok);
            const float g = -expf(a.A_log[h2]) * softplus_f(al + a.dt_bias[h2]);
            rb[(hh * TT + t) * 2 + 0] = expf(g);
            rb[(hh * TT + t) * 2 + 1] = be;
        }
        __syncthreads();
        // ---- optional q/k scaling, and k . q (one wave per token)
        for (int t = wave; t < nt; t += nwaves) {
            constexpr int E = D / 64;
            float qv[E], kv[E];
            float dq = 0.f;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                qv[e] = qs[t * D + lane + 64 * e];
                kv[e] = ks[t * D + lane + 64 * e];
            }
            if constexpr (QKN) {
                float nq = 0.f, nk = 0.f;
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    nq += qv[e] * qv[e];
                    nk += kv[e] * kv[e];
                }
                nq = wave_sum(nq);
                nk = wave_sum(nk);
                const float sq = 1.0f / sqrtf(nq + 1e-6f) / sqrtf((float)D);
                const float sk = 1.0f / sqrtf(nk + 1e-6f);
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    qv[e] *= sq;
                    kv[e] *= sk;
                    qs[t * D + lane + 64 * e] = qv[e];
                    ks[t * D + lane + 64 * e] = kv[e];
                }
            }
#pragma unroll
            for (int e = 0; e < E; ++e) dq += qv[e] * kv[e];
            dq = wave_sum(dq);
            if (lane == 0) kqs[t] = dq;
        }
        __syncthreads();

        // ---- the recurrence over the tile's tokens, state in registers.  Nothing but capture
        // stores touches global memory in this loop; draining the loads first keeps the
        // compiler from placing a full vmcnt wait (which would also wait for the stores) in it.
        __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0)
#pragma unroll 1
        for (int t = 0; t < nt; ++t) {
            // p = S k and S q, accumulated chunk by chunk to keep few values live
            float pk[G::RPL], pq[G::RPL];
#pragma unroll
            for (int i = 0; i < G::RPL; ++i) pk[i] = pq[i] = 0.f;
#pragma unroll
            for (int c4 = 0; c4 < G::NC4; ++c4) {
                const f4 kk = *reinterpret_cast<const f4 *>(ks + t * D + 64 * c4 + 4 * cg);
                const f4 qq = *reinterpret_cast<const f4 *>(qs + t * D + 64 * c4 + 4 * cg);
#pragma unroll
                for (int i = 0; i < G::RPL; ++i)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        pk[i] += S[i][4 * c4 + e] * kk[e];
                        pq[i] += S[i][4 * c4 + e] * qq[e];
                    }
            }
#pragma unroll
            for (int i = 0; i < G::RPL; ++i) {
                pk[i] = row16_sum(pk[i]);
                pq[i] = row16_sum(pq[i]);
            }
            const f2 rbv = *reinterpret_cast<const f2 *>(rb + (hl * TT + t) * 2);
            const float rho = rbv[0], be = rbv[1];
            const float kq = kqs[t];
            const float *vsrc = vs + (hl * TT + t) * D + wih * G::RPW + rg * G::RPL;
#pragma unroll
            for (int i = 0; i < G::RPL; ++i) {
                const float u = be * (vsrc[i] - rho * pk[i]);
                pq[i] = rho * pq[i] + kq * u;  // o = S_new q for row i
                pk[i] = u;
            }
            if (cg == 0) {
                float *od = os + (hl * TT + t) * D + wih * G::RPW + rg * G::RPL;
#pragma unroll
                for (int i = 0; i < G::RPL; ++i) od[i] = pq[i];
            }
#pragma unroll
            for (int c4 = 0; c4 < G::NC4; ++c4) {
                const f4 kk = *reinterpret_cast<const f4 *>(ks + t * D + 64 * c4 + 4 * cg);
#pragma unroll
                for (int i = 0; i < G::RPL; ++i)
#pragma unroll
                    for (int e = 0; e < 4; ++e)  // S <- rho S + u k^T, scaled in place then accumulated
                        S[i][4 * c4 + e] = __builtin_fmaf(pk[i], kk[e], S[i][4 * c4 + e] * rho);
            }
            if constexpr (CAP) {
                float *cp = cap_ptr + (size_t)(t0 + t) * cap_tstride;
#pragma unroll
                for (int i = 0; i < G::RPL; ++i)
#pragma unroll
                    for (int c4 = 0; c4 < G::NC4; ++c4) {
                        const f4 v = {S[i][4 * c4], S[i][4 * c4 + 1], S[i][4 * c4 + 2], S[i][4 * c4 + 3]};
                        store_nt(cp + (size_t)(4 * i) * D + 64 * c4, v);
                    }
            }
        }
        __syncthreads();

        // ---- epilogue: out = o / sqrt(mean(o^2) + eps) * norm_w * silu(z), 16 lanes per row
        {
            constexpr int EPL = D / 16;
            const int grp = tid >> 4, ngrp = nthr >> 4;
#pragma unroll 1
            for (int row = grp; row < R * nt; row += ngrp) {
                const int hh = row / nt, t = row % nt, h2 = hk * R + hh;
                const float *osrc = os + (hh * TT + t) * D;
                float ov[EPL];
                float ss = 0.f;
#pragma unroll
                for (int e = 0; e < EPL; ++e) {
                    ov[e] = osrc[G::perm(cg * EPL + e)];
                    ss += ov[e] * ov[e];
                }
                ss = row16_sum(ss);
                const float inv = 1.0f / sqrtf(ss / (float)D + a.eps);
                const size_t base = (((size_t)b * T + t0 + t) * a.n_vh + h2) * D + cg * EPL;
#pragma unroll
                for (int e = 0; e < EPL; ++e) {
                    const float zz = load_act<ACT_BF16>(a.z, base + e);
                    const float y = ov[e] * inv * a.norm_w[cg * EPL + e] * (zz * sigmoid_f(zz));
                    if constexpr (OUT_BF16)
                        static_cast<uint16_t *>(a.out)[base + e] = f32_to_bf16(y);
                    else
                        static_cast<float *>(a.out)[base + e] = y;
                }
            }
        }
    }

    // ---- final state and conv state (each conv channel is updated by the thread that read it)
    float *sp = a.state + ((size_t)s * a.n_vh + h) * hd + (size_t)row0 * D + cg * 4;
#pragma unroll
    for (int i = 0; i < G::RPL; ++i)
#pragma unroll
        for (int c4 = 0; c4 < G::NC4; ++c4) {
            const f4 v = {S[i][4 * c4], S[i][4 * c4 + 1], S[i][4 * c4 + 2], S[i][4 * c4 + 3]};
            *reinterpret_cast<f4 *>(sp + (size_t)(4 * i) * D + 64 * c4) = v;
        }
    for (int lc = tid; lc < nch; lc += nthr) {
        const int gc = lc < D ? q0 + lc : (lc < 2 * D ? k0 + (lc - D) : v0 + (lc - 2 * D));
        const float r0 = xext(T, gc), r1 = xext(T + 1, gc), r2 = xext(T + 2, gc);
        cs_s[gc] = r0;
        cs_s[(size_t)C + gc] = r1;
        cs_s[(size_t)2 * C + gc] = r2;
    }
}

int verify_waves_per_head(int d) { return d == 128 ? WavesPerHead<128>::value : WavesPerHead<64>::value; }

size_t verify_chain_lds_bytes(int d, int ratio)
{
    const size_t TT = kTokenTile;
    return sizeof(float) * (2 * TT * d + 2 * (size_t)ratio * TT * d + 2 * (size_t)ratio * TT + TT);
}

template <int D, bool AB, bool OB, bool QKN, bool CAP>
static hipError_t launch_t(const VerifyArgs &a, hipStream_t stream)
{
    const int R = a.n_vh / a.n_kh;
    const int threads = R * WavesPerHead<D>::value * 64;
    const size_t lds = verify_chain_lds_bytes(D, R);
    hipLaunchKernelGGL((verify_chain_kernel<D, AB, OB, QKN, CAP>), dim3(a.n_batch * a.n_kh), dim3(threads),
                       lds, stream, a);
    return hipGetLastError();
}

template <int D, bool AB, bool OB, bool QKN>
static hipError_t launch_cap(const VerifyArgs &a, hipStream_t s)
{
    return a.cap_ssm ? launch_t<D, AB, OB, QKN, true>(a, s) : launch_t<D, AB, OB, QKN, false>(a, s);
}
template <int D, bool AB, bool OB>
static hipError_t launch_qkn(const VerifyArgs &a, const LaunchCfg &c, hipStream_t s)
{
    return c.qk_norm ? launch_cap<D, AB, OB, true>(a, s) : launch_cap<D, AB, OB, false>(a, s);
}
template <int D, bool AB>
static hipError_t launch_ob(const VerifyArgs &a, const LaunchCfg &c, hipStream_t s)
{
    return c.out_bf16 ? launch_qkn<D, AB, true>(a, c, s) : launch_qkn<D, AB, false>(a, c, s);
}
template <int D>
static hipError_t launch_ab(const VerifyArgs &a, const LaunchCfg &c, hipStream_t s)
{
    return c.act_bf16 ? launch_ob<D, true>(a, c, s) : launch_ob<D, false>(a, c, s);
}

hipError_t launch_verify_chain(const VerifyArgs &a, const LaunchCfg &c, hipStream_t stream)
{
    if (a.d == 128) return launch_ab<128>(a, c, stream);
    if (a.d == 64) return launch_ab<64>(a, c, stream);
    return hipErrorInvalidValue;
}

}  // namespace gdn
