// gdn_geo.h - register layout of one value head's d_v x d_k fp32 state across a workgroup.
//
//   lane = 16 * rg + cg,  rg in [0,4) picks a row group, cg in [0,16) a column group
//   rows  of register i : wave_in_head * 4*RPL + 4*i + rg          (RPL rows per lane)
//   cols  of chunk c4   : 64*c4 + 4*cg + e,  e in [0,4)             (CPL = d/16 columns)
// One float4 store instruction covers 4 consecutive rows x 64 contiguous columns, so every
// 128-byte line of a state snapshot is written whole by a single instruction; contractions over
// the key index finish with a 16-lane DPP sum.
#pragma once

#include "gdn_device.h"

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

    // One token of the gated delta rule for the state rows one lane holds (layout above), shared by
    // the chain and tree kernels so that the same token sequence gives the same bits in both:
    //   p = S k,  u = beta (v - rho p),  S <- rho S + u k^T,  o = rho (S_old q) + (k . q) u  (= S_new q)
    // krow, qrow: the token's k and q in LDS (natural column order); vrow: its v at this lane's rows
    // (perm order).  k . q and, with QKN, the q / k norms come from the same 16-lane sums as S k:
    // k^ = k / |k|, q^ = q / |q| / sqrt(d) enter as scale factors.  Writes o for the lane's rows.
    template <bool QKN>
    __device__ static __forceinline__ void step(float (&S)[RPL][CPL], const float *krow, const float *qrow,
                                                const float *vrow, float rho, float bet, int cg, float (&o)[RPL])
    {
        float pk[RPL], pq[RPL];
        float kq = 0.f, nk = 0.f, nq = 0.f;
#pragma unroll
        for (int i = 0; i < RPL; ++i) pk[i] = pq[i] = 0.f;
#pragma unroll
        for (int c4 = 0; c4 < NC4; ++c4) {
            const f4 kk = *reinterpret_cast<const f4 *>(krow + 64 * c4 + 4 * cg);
            const f4 qq = *reinterpret_cast<const f4 *>(qrow + 64 * c4 + 4 * cg);
#pragma unroll
            for (int i = 0; i < RPL; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    pk[i] += S[i][4 * c4 + e] * kk[e];
                    pq[i] += S[i][4 * c4 + e] * qq[e];
                }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                kq += kk[e] * qq[e];
                if constexpr (QKN) {
                    nk += kk[e] * kk[e];
                    nq += qq[e] * qq[e];
                }
            }
        }
#pragma unroll
        for (int i = 0; i < RPL; ++i) {
            pk[i] = row16_sum(pk[i]);
            pq[i] = row16_sum(pq[i]);
        }
        kq = row16_sum(kq);
        float sk = 1.f;  // scale of the raw k row in the update
        if constexpr (QKN) {
            sk = rsqrt_f(row16_sum(nk) + 1e-6f);
            const float sq = rsqrt_f(row16_sum(nq) + 1e-6f) * (1.0f / sqrtf((float)D));
#pragma unroll
            for (int i = 0; i < RPL; ++i) {
                pk[i] *= sk;
                pq[i] *= sq;
            }
            kq *= sk * sq;
        }
#pragma unroll
        for (int i = 0; i < RPL; ++i) {
            const float u = bet * (vrow[i] - rho * pk[i]);
            o[i] = rho * pq[i] + kq * u;
            pk[i] = u * sk;
        }
#pragma unroll
        for (int c4 = 0; c4 < NC4; ++c4) {
            const f4 kk = *reinterpret_cast<const f4 *>(krow + 64 * c4 + 4 * cg);
#pragma unroll
            for (int i = 0; i < RPL; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e)  // S <- rho S + u k^T, scaled in place then accumulated
                    S[i][4 * c4 + e] = __builtin_fmaf(pk[i], kk[e], S[i][4 * c4 + e] * rho);
        }
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

}  // namespace gdn
