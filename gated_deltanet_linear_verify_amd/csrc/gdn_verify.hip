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
// contractions over the key index (S k, S q and k . q) finish with a 16-lane DPP sum.
//
// Per token (Yang, Kautz & Hatamizadeh 2024, gated delta rule; Geo::step, shared with the tree kernel):
//   p = S k,  u = beta (v - rho p),  S <- rho S + u k^T,  o = rho (S_old q) + (k.q) u  (= S_new q)
// The capture of S after every token (lucebox-hub internal.h, struct TargetCache,
// ssm_intermediate) streams out while the next token is computed; the RMS norm + SiLU(z)
// epilogue (ssm_norm, z projection: internal.h, struct TargetLayer) runs per token tile.
//
// Memory schedule.  gfx950 has one vector-memory counter for loads and stores, so a load issued
// after the capture stores would have to wait for them.  A launch therefore stages everything it
// reads (raw qkv rows and z straight into LDS with global_load_lds, alpha, beta, conv taps, conv
// state and the recurrent state into registers) before the token loop; the token loop and the
// epilogue only read LDS and only store to global memory.  One launch covers up to 16 tokens;
// longer chains are consecutive launches that pick up the state the previous one left.
#include "gdn_device.h"
#include "gdn_geo.h"
#include "gdn_internal.h"

#include <type_traits>

namespace gdn {

// Capture stores stream past the caches (store_stream): the 2 GiB capture is written once and only
// the rollback's few positions are read back.
__device__ __forceinline__ void store_cap(float *p, f4 v) { store_stream(p, v); }

// Occupancy cap: about 8 waves per CU.  The capture stream writes faster with fewer concurrent
// write streams per CU (measured: ~5.9 vs ~5.6 TB/s for the bare store pattern), and 2 waves per
// SIMD still hide the token loop's arithmetic under the stores.  The cap is applied by requesting
// enough LDS that no more workgroups fit on a CU (160 KiB of LDS per CU).
constexpr size_t kLdsPerCu = 160 * 1024;
constexpr int kTargetWavesPerCu = 8;

// LDS carve-up of one workgroup (R value heads in the workgroup, act_t = activation storage type).
template <int D, typename act_t>
struct VerifyLds {
    static constexpr int TT = kTokenTile;
    __host__ __device__ static size_t raw_bytes(int R) { return (size_t)TT * (2 + R) * D * sizeof(act_t); }
    __host__ __device__ static size_t o_bytes(int R) { return (size_t)R * TT * D * sizeof(float); }
    __host__ __device__ static size_t region(int R) { return raw_bytes(R) > o_bytes(R) ? raw_bytes(R) : o_bytes(R); }
    __host__ __device__ static size_t total(int R)
    {
        return sizeof(float) * (2 * TT * D + (size_t)R * TT * D)  // ks, qs, vs
               + region(R)                                          // os, aliased by the raw rows
               + (size_t)R * TT * D * sizeof(act_t)                 // zs
               + sizeof(float) * (2 * (size_t)R * TT + TT + D);      // rb, (pad), norm_w
    }
};

// One (token, value head) row of the output, out = o / sqrt(mean(o^2) + eps) * norm_w * silu(z),
// worked by 16 lanes: lane cg holds o at rows cg EPL .. cg EPL + EPL - 1 (ov), the matching z and
// norm weights.  Shared by the fused epilogue and the row-split norm kernel, which therefore give
// the same bits.
template <bool OUT_BF16, int D>
__device__ __forceinline__ void norm_gate_vals(const float (&ov)[D / 16], const float *nwr, const float (&zv)[D / 16],
                                               float eps, void *out, size_t base)
{
    constexpr int EPL = D / 16;
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) ss += ov[e] * ov[e];
    ss = row16_sum(ss);
    const float inv = 1.0f / sqrtf(ss / (float)D + eps);
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
        const float zz = zv[e];
        const float y = ov[e] * inv * nwr[e] * (zz * sigmoid_f(zz));
        if constexpr (OUT_BF16)
            static_cast<uint16_t *>(out)[base + e] = f32_to_bf16(y);
        else
            static_cast<float *>(out)[base + e] = y;
    }
}
template <bool ACT_BF16, bool OUT_BF16, int D>
__device__ __forceinline__ void norm_gate_row(const float (&ov)[D / 16], const float *nwr,
                                              const typename std::conditional<ACT_BF16, uint16_t, float>::type *zrow,
                                              float eps, void *out, size_t base)
{
    float zv[D / 16];
#pragma unroll
    for (int e = 0; e < D / 16; ++e) {
        if constexpr (ACT_BF16)
            zv[e] = bf16_to_f32(zrow[e]);
        else
            zv[e] = zrow[e];
    }
    norm_gate_vals<OUT_BF16, D>(ov, nwr, zv, eps, out, base);
}

// Row split (SPLIT): kRowSplit workgroups per value head, each with NW waves that hold its share of
// the head's rows in the layout of NW * kRowSplit waves (so every row sees the same arithmetic as
// in one workgroup).  A workgroup writes its rows' state, capture and v conv; its readout goes to
// the scratch, and verify_norm_kernel applies the norm and gate, and writes the q / k conv, after
// the launch.  One token's state update over a d x d head is ~d^2 fused multiply-adds per
// contraction, which one CU's vector units take ~1000 clocks for at d = 128: splitting the rows
// over CUs is what shortens the token chain when few heads are in flight.
constexpr int kRowSplit = 4;

// The row split's scratch: its readout [n_batch][16][H_v][d], then the q / k channels' starting rows
// (the three conv rows a launch begins from) [n_batch][3][2 H_k d].
__device__ __forceinline__ float *split_qk_rows(const VerifyArgs &a, int b)
{
    return a.oscr + (size_t)a.n_batch * kTokenTile * a.n_vh * a.d + (size_t)b * 3 * 2 * a.n_kh * a.d;
}

// NW: waves per value head (4 at d = 128 with all of a key head's value heads in the workgroup,
// 8 with one value head per workgroup: half the rows per lane, the same arithmetic per row), or
// per workgroup of a row split.
template <int D, bool ACT_BF16, bool OUT_BF16, bool QKN, bool CAP, int NW, bool SPLIT>
__global__ __launch_bounds__(1024) void verify_chain_kernel(VerifyArgs a)
{
    using act_t = typename std::conditional<ACT_BF16, uint16_t, float>::type;
    using L = VerifyLds<D, act_t>;
    using G = Geo<D, SPLIT ? NW * kRowSplit : NW>;
    constexpr int TT = kTokenTile;
    constexpr int VEC = 16 / (int)sizeof(act_t);  // activations per 16-byte load
    const int R = a.n_vh / a.n_kh;  // value heads per key head
    const int HW = SPLIT ? 1 : a.hpw;  // value heads of this workgroup: R, or 1 (few batch entries)
    const int nthr = blockDim.x;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int nwaves = nthr >> 6;
    const int rj = SPLIT ? blockIdx.x % kRowSplit : 0;  // this workgroup's share of a split head
    const int wgi = SPLIT ? blockIdx.x / kRowSplit : blockIdx.x;
    const int hl = SPLIT ? 0 : wave / NW, wih = SPLIT ? rj * NW + wave : wave % NW;
    const int rg = lane >> 4, cg = lane & 15;

    const int gpb = a.n_vh / HW;       // workgroups (sets of a split) per batch entry
    const int b = wgi / gpb;
    const int h0 = (wgi % gpb) * HW;  // first value head of the workgroup
    const int hk = h0 / R;
    const int h = h0 + hl;
    // With one value head per workgroup the key head's q / k channels are shared, and every
    // workgroup of the key head reads their starting rows here, so none of them writes those
    // channels: qk_conv_state_kernel writes their conv window rows and conv state after the launch.
    const bool own_qk = HW == R && !SPLIT;
    const int s = a.slot_ids[b];
    if (s < 0 || s >= a.n_pool) return;  // uniform over the workgroup
    // A rollback left pending by the previous round: the first launch of the call starts from the
    // state after capture position ra of this same capture, written by that round's verify, instead
    // of from the slot's state.  This workgroup reads only its own heads' and channels' slices of
    // position ra, and every read lands before its first capture store.
    // With the commit deferred, a launch after the first continues from the previous launch's last
    // capture position in the same way, since the state buffer is not written.
    int ra = -1;
    if constexpr (CAP) {
        if (a.resume) {
            const int r = a.resume[b];
            if (r >= a.t_cap) return;  // outside the capture: every launch skips the entry (uniform)
            if (a.t0 == 0) ra = r;
        }
        if (a.defer && a.t0 > 0) ra = a.t0 - 1;
    }
    const bool commit = !(CAP && a.defer);  // write the state and conv state after the last token

    extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
    float *ks = reinterpret_cast<float *>(smem_raw);  // [TT][D]
    float *qs = ks + TT * D;                            // [TT][D]
    float *vs = qs + TT * D;                            // [HW][TT][D]  rows in perm order
    float *os = vs + HW * TT * D;                       // [HW][TT][D]  rows in perm order
    act_t *raw = reinterpret_cast<act_t *>(os);         // [TT][nch]    staged qkv rows (prologue only)
    act_t *zs = reinterpret_cast<act_t *>(reinterpret_cast<unsigned char *>(os) + L::region(HW));  // [TT][HW*D]
    float *rb = reinterpret_cast<float *>(zs + HW * TT * D);  // [HW][TT][2]  (rho, beta)
    float *nws = rb + HW * TT * 2 + TT;                         // [D]          norm_w

    const int C = a.C;
    const int T = a.T;    // tokens of the whole call: the row stride of qkv, z, alpha, beta, out
    const int t0 = a.t0;  // first token of this launch
    const int nt = a.nt;  // tokens of this launch, 1 .. TT
    const int nch = (2 + HW) * D;
    const int q0 = hk * D, k0 = a.n_kh * D + hk * D, v0 = 2 * a.n_kh * D + h0 * D;
    float *cs_s = a.conv_state + (size_t)s * 3 * C;
    // conv state the launch starts from: the slot's, or capture window rows ra+1 .. ra+3
    const float *cs_src = ra >= 0 ? a.cap_conv + ((size_t)s * (3 + a.t_cap) + ra + 1) * C : cs_s;
    const size_t hd = (size_t)D * D;
    const act_t *qkv_b = static_cast<const act_t *>(a.qkv) + ((size_t)b * T + t0) * C;
    const act_t *z_b = static_cast<const act_t *>(a.z) + ((size_t)b * T + t0) * a.n_vh * D + (size_t)h0 * D;
    auto to_f32 = [](act_t x) -> float {
        if constexpr (ACT_BF16)
            return bf16_to_f32(x);
        else
            return x;
    };
    // local channel -> global channel of the fused qkv stream (blocks q | k | v)
    auto gchan = [&](int lc) -> int { return lc < D ? q0 + lc : (lc < 2 * D ? k0 + (lc - D) : v0 + (lc - 2 * D)); };

    // ================= stage: every global load of the launch is issued up front =================
    // The qkv rows go straight from HBM into LDS (global_load_lds_dwordx4: lane i of a wave lands
    // at the wave's LDS base + 16 i) in row-major [token][local channel] order: no VGPR holds them.
    const int nvr = nch / VEC;  // 16-byte vectors per staged row
    for (int it = tid; it < nt * nvr; it += nthr) {
        const int r = it / nvr, lc = (it % nvr) * VEC;
        lds_dma16(qkv_b + (uint32_t)(r * C + gchan(lc)), raw + it * VEC);
    }
    // z: [nt][HW*D] is contiguous in HBM and in LDS
    for (int it = tid; it < nt * HW * D / VEC; it += nthr) {
        const int e0 = it * VEC, t = e0 / (HW * D), within = e0 % (HW * D);
        lds_dma16(z_b + (uint32_t)(t * a.n_vh * D + within), zs + e0);
    }
    // alpha and beta: at most one (token, head) per thread of the last nt * HW threads (with one
    // value head per workgroup their wave has no conv channel, so the gates overlap the conv), with
    // the head's A_log and dt_bias.  The loads sit outside any branch (the other threads load a
    // valid entry they never use) and nothing is computed from them before the wait below: a bf16
    // conversion, or a branch join over a loaded register, would make the compiler wait for every
    // load issued so far, the qkv and z transfers included, before the state loads even start.
    const int gate_t0 = nthr - nt * HW;  // the first gate thread
    const int ab_i = min(max(tid - gate_t0, 0), nt * HW - 1);
    const int ab_h = h0 + ab_i % HW;
    const size_t ab_tok = ((size_t)b * T + t0 + ab_i / HW) * a.n_vh + ab_h;
    using word_t = typename std::conditional<ACT_BF16, uint16_t, uint32_t>::type;  // bf16 or fp32 bits
    uint32_t al_raw = static_cast<const word_t *>(a.alpha)[ab_tok];
    uint32_t be_raw = static_cast<const word_t *>(a.beta)[ab_tok];
    float alog = a.A_log[ab_h], dtb = a.dt_bias[ab_h];
    // The channels this workgroup convolves: q, k and its heads' v; in a row split only the v
    // channels of its own rows, which no other workgroup of the split reads or writes (the others'
    // v rows are written during the launch, as its own are).
    auto conv_chan = [&](int lc) {
        return lc < nch && (!SPLIT || lc < 2 * D || (lc - 2 * D) / (D / kRowSplit) == rj);
    };
    // conv taps and the slot's conv state (xext rows 0..2 of the launch) of this thread's channels
    f4 wv[2];
    float csv[2][3];
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int lc = tid + it * nthr;
        if (conv_chan(lc)) {
            const int gc = gchan(lc);
            wv[it] = *reinterpret_cast<const f4 *>(a.conv_w + (size_t)gc * 4);
#pragma unroll
            for (int r = 0; r < 3; ++r) csv[it][r] = cs_src[(uint32_t)(r * C + gc)];
        }
    }
    // the recurrent state, into registers
    float S[G::RPL][G::CPL];  // S[i][4 c4 + e] = state row (row0 + 4 i), column (64 c4 + 4 cg + e)
    const int row0 = wih * G::RPW + rg;
    const float *st_src = ra >= 0 ? a.cap_ssm + (((size_t)s * a.t_cap + ra) * a.n_vh + h) * hd
                                  : a.state + ((size_t)s * a.n_vh + h) * hd;
    const float *st_ptr = st_src + (size_t)row0 * D + cg * 4;
#pragma unroll
    for (int i = 0; i < G::RPL; ++i)
#pragma unroll
        for (int c4 = 0; c4 < G::NC4; ++c4) {
            const f4 v = *reinterpret_cast<const f4 *>(st_ptr + (size_t)(4 * i) * D + 64 * c4);
#pragma unroll
            for (int e = 0; e < 4; ++e) S[i][4 * c4 + e] = v[e];
        }
    float nw = a.norm_w[min(tid, D - 1)];
    __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0): registers loaded, LDS rows landed
    asm volatile("" : "+v"(al_raw), "+v"(be_raw), "+v"(alog), "+v"(dtb), "+v"(nw));  // nothing above
    if constexpr (SPLIT) {
        // the key head's q / k starting rows, for the kernel after the launch (split_qk_rows): written
        // by one workgroup of the key head, indexed by batch entry so that it reads them unconditionally
        if (rj == 0 && h % R == 0 && tid < 2 * D) {
            float *qk = split_qk_rows(a, b) + gchan(tid);
#pragma unroll
            for (int r = 0; r < 3; ++r) qk[(size_t)r * 2 * a.n_kh * D] = csv[0][r];
        }
    }
    auto word_f32 = [](uint32_t w) -> float {
        if constexpr (ACT_BF16)
            return bf16_to_f32((uint16_t)w);
        else
            return __builtin_bit_cast(float, w);
    };
    if (tid < D) nws[tid] = nw;
    __syncthreads();  // the staged rows of every wave have landed
    if (tid >= gate_t0) {  // rho and beta per (token, head), read only after the conv's barrier
        const int t = ab_i / HW, hh = ab_i % HW;
        const float g = -expf(alog) * softplus_f(word_f32(al_raw) + dtb);
        rb[(hh * TT + t) * 2 + 0] = expf(g);
        rb[(hh * TT + t) * 2 + 1] = word_f32(be_raw);
    }

    // ================= depthwise causal conv (one thread per channel) =================
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int lc = tid + it * nthr;
        if (conv_chan(lc)) {
            const int gc = gchan(lc);
            float *dst;
            if (lc < D)
                dst = qs + lc;
            else if (lc < 2 * D)
                dst = ks + (lc - D);
            else
                dst = vs + ((lc - 2 * D) / D) * TT * D + G::perm((lc - 2 * D) % D);
            // the window: the starting rows, then the launch's raw rows, every LDS read issued before
            // any tap sum (rows past nt lie inside the staging area and are never used)
            float x[TT + 3];
            x[0] = csv[it][0];
            x[1] = csv[it][1];
            x[2] = csv[it][2];
#pragma unroll
            for (int t = 0; t < TT; ++t) x[t + 3] = to_f32(raw[t * nch + lc]);
            const f4 w = wv[it];
            const bool own = lc >= 2 * D || own_qk;  // this workgroup writes the channel's rows
            float *cc = CAP ? a.cap_conv + (size_t)s * (3 + a.t_cap) * C + gc : nullptr;
            if (CAP && t0 == 0 && own) {  // the window starts with the conv state the call began from
                cc[0] = x[0];
                cc[(size_t)C] = x[1];
                cc[(size_t)2 * C] = x[2];
            }
            // every row of the tile is convolved and written (rows past nt are never read)
#pragma unroll
            for (int t = 0; t < TT; ++t) {
                float y = conv4(w, x[t], x[t + 1], x[t + 2], x[t + 3]);
                if constexpr (QKN) y = y * sigmoid_f(y);
                dst[t * D] = y;
            }
            if (CAP && own) {
#pragma unroll
                for (int t = 0; t < TT; ++t)
                    if (t < nt) cc[(size_t)(t0 + t + 3) * C] = x[t + 3];
            }
            float e0 = x[0], e1 = x[1], e2 = x[2];  // window rows nt .. nt + 2: the conv state after the launch
#pragma unroll
            for (int t = 1; t <= TT; ++t) {
                e0 = t == nt ? x[t] : e0;
                e1 = t == nt ? x[t + 1] : e1;
                e2 = t == nt ? x[t + 2] : e2;
            }
            // this thread was the only reader of these elements
            if (commit && own) {
                cs_s[gc] = e0;
                cs_s[(size_t)C + gc] = e1;
                cs_s[(size_t)2 * C + gc] = e2;
            }
        }
    }
    __syncthreads();
    // ================= the recurrence, state in registers =================
    // Only LDS reads and capture stores from here on: no wait on the memory counter, which the
    // capture stores occupy.
    float *cap_ptr = nullptr;
    size_t cap_tstride = 0;
    if constexpr (CAP) {
        cap_ptr = a.cap_ssm + (((size_t)s * a.t_cap + t0) * a.n_vh + h) * hd + (size_t)row0 * D + cg * 4;
        cap_tstride = (size_t)a.n_vh * hd;
    }
#pragma unroll 1
    for (int t = 0; t < nt; ++t) {
        const f2 rbv = *reinterpret_cast<const f2 *>(rb + (hl * TT + t) * 2);
        float o[G::RPL];
        G::template step<QKN>(S, ks + t * D, qs + t * D, vs + (hl * TT + t) * D + wih * G::RPW + rg * G::RPL, rbv[0],
                              rbv[1], cg, o);
        if (cg == 0) {
            float *od = os + (hl * TT + t) * D + wih * G::RPW + rg * G::RPL;
#pragma unroll
            for (int i = 0; i < G::RPL; ++i) od[i] = o[i];
        }
        if constexpr (CAP) {
            float *cp = cap_ptr + (size_t)t * cap_tstride;
#pragma unroll
            for (int i = 0; i < G::RPL; ++i)
#pragma unroll
                for (int c4 = 0; c4 < G::NC4; ++c4) {
                    const f4 v = {S[i][4 * c4], S[i][4 * c4 + 1], S[i][4 * c4 + 2], S[i][4 * c4 + 3]};
                    store_cap(cp + (size_t)(4 * i) * D + 64 * c4, v);
                }
        }
    }
    // ---- final state (address rebuilt from a wave-uniform base so none is kept across the loop)
    if (commit) {
        uint32_t off = (uint32_t)(row0 * D + cg * 4);
        asm volatile("" : "+v"(off));
        float *sp = a.state + ((size_t)s * a.n_vh + h) * hd;
#pragma unroll
        for (int i = 0; i < G::RPL; ++i)
#pragma unroll
            for (int c4 = 0; c4 < G::NC4; ++c4) {
                const f4 v = {S[i][4 * c4], S[i][4 * c4 + 1], S[i][4 * c4 + 2], S[i][4 * c4 + 3]};
                *reinterpret_cast<f4 *>(sp + off + (uint32_t)(4 * i * D + 64 * c4)) = v;
            }
    }
    lds_barrier();  // o of every head is in LDS; the capture stores stay in flight

    if constexpr (SPLIT) {
        // ================= the readout of this workgroup's rows, natural row order, to the scratch
        constexpr int RW = D / kRowSplit;
        for (int i = tid; i < nt * RW; i += nthr) {
            const int t = i / RW, r = rj * RW + i % RW;
            a.oscr[(((size_t)b * TT + t) * a.n_vh + h) * D + r] = os[t * D + G::perm(r)];
        }
        return;
    }
    // ================= epilogue: out = o / sqrt(mean(o^2) + eps) * norm_w * silu(z) =================
    constexpr int EPL = D / 16;  // 16 lanes per (head, token) row
    const int grp = tid >> 4, ngrp = nthr >> 4;
#pragma unroll 1
    for (int row = grp; row < HW * nt; row += ngrp) {
        const int hh = row / nt, t = row % nt, h2 = h0 + hh;
        const float *osrc = os + (hh * TT + t) * D;
        float ov[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) ov[e] = osrc[G::perm(cg * EPL + e)];
        const size_t base = (((size_t)b * T + t0 + t) * a.n_vh + h2) * D + cg * EPL;
        norm_gate_row<ACT_BF16, OUT_BF16, D>(ov, nws + cg * EPL, zs + t * HW * D + hh * D + cg * EPL, a.eps, a.out,
                                             base);
    }
}

int verify_waves_per_head(int d) { return d == 128 ? WavesPerHead<128>::value : WavesPerHead<64>::value; }

size_t verify_chain_lds_bytes(int d, int ratio, bool act_bf16)
{
    if (d == 128) return act_bf16 ? VerifyLds<128, uint16_t>::total(ratio) : VerifyLds<128, float>::total(ratio);
    return act_bf16 ? VerifyLds<64, uint16_t>::total(ratio) : VerifyLds<64, float>::total(ratio);
}

// The key heads' q / k channels after a launch that ran one value head per workgroup: their conv
// window rows of the launch (with capture) and their conv state after it (unless the commit is
// deferred).  The launch's conv input is its starting rows (the slot's conv state, or the capture
// window rows it resumes from, chosen as in the verify kernel) followed by its tokens.  Every read
// of a channel precedes its writes, and all of them are issued before the first is used.
// STASH (after a row split): the starting rows come from split_qk_rows, written by the launch, and
// every load is issued before the batch entry's slot is known, so the kernel waits for memory once.
template <bool ACT_BF16, bool CAP, bool STASH = false>
__device__ __forceinline__ void qk_conv_channel(const VerifyArgs &a, int b, int ch)
{
    using act_t = typename std::conditional<ACT_BF16, uint16_t, float>::type;
    if (ch >= 2 * a.n_kh * a.d) return;  // q | k channels are 0 .. 2 H_k d - 1
    const size_t C = (size_t)a.C;
    const int t0 = a.t0, nt = a.nt;
    const act_t *x = static_cast<const act_t *>(a.qkv) + ((size_t)b * a.T + t0) * C + ch;
    float xs[3 + kTokenTile];
    act_t tok[kTokenTile];
    if constexpr (STASH) {
        const float *st = split_qk_rows(a, b) + ch;
#pragma unroll
        for (int r = 0; r < 3; ++r) xs[r] = st[(size_t)r * 2 * a.n_kh * a.d];
#pragma unroll
        for (int t = 0; t < kTokenTile; ++t) tok[t] = x[(size_t)(t < nt ? t : nt - 1) * C];  // valid rows only
    }
    const int s = a.slot_ids[b];
    if (s < 0 || s >= a.n_pool) return;  // uniform over the block, as in the verify kernel
    int ra = -1;
    if constexpr (CAP) {
        if (a.resume) {
            const int r = a.resume[b];
            if (r >= a.t_cap) return;  // skipped by the verify kernel too
            if (a.t0 == 0) ra = r;
        }
        if (a.defer && a.t0 > 0) ra = a.t0 - 1;
    }
    const bool commit = !(CAP && a.defer);
    float *cs = a.conv_state + (size_t)s * 3 * C + ch;
    float *cw = CAP ? a.cap_conv + (size_t)s * (3 + a.t_cap) * C + ch : nullptr;
    if constexpr (!STASH) {
        const float *src = ra >= 0 ? cw + (size_t)(ra + 1) * C : cs;
#pragma unroll
        for (int r = 0; r < 3; ++r) xs[r] = src[(size_t)r * C];
#pragma unroll
        for (int t = 0; t < kTokenTile; ++t) tok[t] = x[(size_t)(t < nt ? t : nt - 1) * C];  // valid rows only
    }
#pragma unroll
    for (int t = 0; t < kTokenTile; ++t) {
        if constexpr (ACT_BF16)
            xs[3 + t] = bf16_to_f32(tok[t]);
        else
            xs[3 + t] = tok[t];
    }
    if constexpr (CAP) {
        if (t0 == 0)
#pragma unroll
            for (int r = 0; r < 3; ++r) cw[(size_t)r * C] = xs[r];
#pragma unroll
        for (int t = 0; t < kTokenTile; ++t)
            if (t < nt) cw[(size_t)(t0 + t + 3) * C] = xs[3 + t];
    }
    if (commit)
#pragma unroll
        for (int r = 0; r < 3; ++r) cs[(size_t)r * C] = xs[nt + r];
}
template <bool ACT_BF16, bool CAP>
__global__ __launch_bounds__(256) void qk_conv_state_kernel(VerifyArgs a)
{
    qk_conv_channel<ACT_BF16, CAP>(a, blockIdx.y, blockIdx.x * blockDim.x + threadIdx.x);
}

// After a row-split launch: its first blocks write the key heads' q / k conv as qk_conv_state_kernel
// does (per batch entry, 256 channels a block), the others apply the norm and gate to the readout
// in the scratch, 16 lanes per (batch entry, token, value head) row, as the fused epilogue does.
template <int D, bool ACT_BF16, bool OUT_BF16, bool CAP>
__global__ __launch_bounds__(256) void verify_norm_kernel(VerifyArgs a)
{
    using act_t = typename std::conditional<ACT_BF16, uint16_t, float>::type;
    constexpr int EPL = D / 16;
    const int conv_blocks = (2 * a.n_kh * D + 255) / 256;
    const int nconv = conv_blocks * a.n_batch;
    if ((int)blockIdx.x < nconv) {
        qk_conv_channel<ACT_BF16, CAP, true>(a, blockIdx.x / conv_blocks, (blockIdx.x % conv_blocks) * 256 + threadIdx.x);
        return;
    }
    // every lane of a 16-lane group takes the same row, so the returns below are uniform per group
    const int row = ((int)blockIdx.x - nconv) * 16 + (int)(threadIdx.x >> 4), cg = threadIdx.x & 15;
    if (row >= a.n_batch * a.nt * a.n_vh) return;
    const int h = row % a.n_vh, t = (row / a.n_vh) % a.nt, b = row / (a.n_vh * a.nt);
    // everything the row needs is indexed by batch entry: loaded before its slot is checked
    const float *o = a.oscr + (((size_t)b * kTokenTile + t) * a.n_vh + h) * D + cg * EPL;
    const size_t base = (((size_t)b * a.T + a.t0 + t) * a.n_vh + h) * D + cg * EPL;
    const act_t *zrow = static_cast<const act_t *>(a.z) + base;
    float ov[EPL], nwr[EPL], zv[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
        ov[e] = o[e];
        nwr[e] = a.norm_w[cg * EPL + e];
        if constexpr (ACT_BF16)
            zv[e] = bf16_to_f32(zrow[e]);
        else
            zv[e] = zrow[e];
    }
    const int s = a.slot_ids[b];
    if (s < 0 || s >= a.n_pool) return;  // skipped by the verify kernel too
    if (CAP && a.resume && a.resume[b] >= a.t_cap) return;
    norm_gate_vals<OUT_BF16, D>(ov, nwr, zv, a.eps, a.out, base);
}

// Value heads per workgroup.  With few batch entries a workgroup per key head leaves most CUs idle
// and each one streams its heads' whole capture through one store path (~64 B per clock), so then
// each value head gets its own workgroup.  Not below 3 tokens: there the second launch costs more
// than the split saves (one slot: 9.4 against 11.1 us at 1 token, even at 2, ahead from 3 on;
// likewise at 4 slots).
constexpr int kSplitMaxWorkgroups = 64;
constexpr int kSplitMinTokens = 3;
static int heads_per_workgroup(const VerifyArgs &a)
{
    const int R = a.n_vh / a.n_kh;
    if (R == 1 || a.T < kSplitMinTokens) return R;
    return (long)a.n_batch * a.n_kh <= kSplitMaxWorkgroups ? 1 : R;
}

// Row split: when the call's value heads times kRowSplit fit one workgroup per CU (one slot of 32
// heads: 128 workgroups), from kSplitMinTokens tokens, and the readout fits the scratch.
constexpr int kCus = 256;
static bool row_split(const VerifyArgs &a)
{
    if (a.T < kSplitMinTokens || (long)a.n_batch * a.n_vh * kRowSplit > kCus) return false;
    return (size_t)a.n_batch * (kTokenTile * a.n_vh + 3 * 2 * a.n_kh) * a.d * sizeof(float) <= kSplitScratchBytes;
}

// One launch covers at most kTokenTile tokens; longer chains are consecutive launches on the same
// stream, each starting from the state and conv state the previous one left.
template <int D, bool AB, bool OB, bool QKN, bool CAP>
static hipError_t launch_t(const VerifyArgs &a0, hipStream_t stream)
{
    const int R = a0.n_vh / a0.n_kh;
    const int HW = heads_per_workgroup(a0);
    const int nw = HW < R ? 2 * WavesPerHead<D>::value : WavesPerHead<D>::value;  // waves per value head
    const int threads = HW * nw * 64;
    size_t lds = verify_chain_lds_bytes(D, HW, AB);
    const int waves = HW * nw;
    const int wgs_per_cu = waves >= kTargetWavesPerCu ? 1 : kTargetWavesPerCu / waves;
    const size_t lds_cap = kLdsPerCu / (wgs_per_cu + 1) + 16;  // wgs_per_cu + 1 workgroups no longer fit
    if (CAP && lds < lds_cap) lds = lds_cap;  // without capture stores more resident waves only help
    float *oscr = row_split(a0) ? static_cast<float *>(split_scratch(stream, true)) : nullptr;
    for (int t0 = 0; t0 < a0.T; t0 += kTokenTile) {
        VerifyArgs a = a0;
        a.t0 = t0;
        a.nt = a0.T - t0 < kTokenTile ? a0.T - t0 : kTokenTile;
        if (oscr) {
            constexpr int NWS = 2 * WavesPerHead<D>::value;  // waves per workgroup of the split
            a.hpw = 1;
            a.oscr = oscr;
            size_t lds1 = verify_chain_lds_bytes(D, 1, AB);
            const size_t cap1 = kLdsPerCu / (kTargetWavesPerCu / NWS + 1) + 16;
            if (CAP && lds1 < cap1) lds1 = cap1;
            hipLaunchKernelGGL((verify_chain_kernel<D, AB, OB, QKN, CAP, NWS, true>),
                               dim3(a.n_batch * a.n_vh * kRowSplit), dim3(NWS * 64), lds1, stream, a);
            if (hipError_t e = hipGetLastError()) return e;
            const unsigned blocks = (unsigned)(((2 * a.n_kh * D + 255) / 256) * a.n_batch +
                                               (a.n_batch * a.nt * a.n_vh + 15) / 16);
            hipLaunchKernelGGL((verify_norm_kernel<D, AB, OB, CAP>), dim3(blocks), dim3(256), 0, stream, a);
            if (hipError_t e = hipGetLastError()) return e;
            continue;
        }
        a.hpw = HW;
        if (HW < R)
            hipLaunchKernelGGL((verify_chain_kernel<D, AB, OB, QKN, CAP, 2 * WavesPerHead<D>::value, false>),
                               dim3(a.n_batch * (a.n_vh / HW)), dim3(threads), lds, stream, a);
        else
            hipLaunchKernelGGL((verify_chain_kernel<D, AB, OB, QKN, CAP, WavesPerHead<D>::value, false>),
                               dim3(a.n_batch * (a.n_vh / HW)), dim3(threads), lds, stream, a);
        if (hipError_t e = hipGetLastError()) return e;
        if (HW < R) {
            const unsigned blocks = (unsigned)((2 * a.n_kh * D + 255) / 256);
            hipLaunchKernelGGL((qk_conv_state_kernel<AB, CAP>), dim3(blocks, a.n_batch), dim3(256), 0, stream, a);
            if (hipError_t e = hipGetLastError()) return e;
        }
    }
    return hipSuccess;
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
