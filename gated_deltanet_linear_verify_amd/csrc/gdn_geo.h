// gdn_geo.h - register layout of one value head's d_v x d_k fp32 state across a workgroup.
//
//   lane = 16 * rg + cg,  rg in [0,4) picks a row group, cg in [0,16) a column group
//   rows  of register i : wave_in_head * 4*RPL + 4*i + rg          (RPL rows per lane)
//   cols  of chunk c4   : 64*c4 + 4*cg + e,  e in [0,4)             (CPL = d/16 columns)
// One float4 store instruction covers 4 consecutive rows x 64 contiguous columns, so every
// 128-byte line of a state snapshot is written whole by a single instruction; contractions over
// the key index finish with a 16-lane DPP sum.
#pragma once

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

}  // namespace gdn
