// gdn_tree.hip - tree verify: every node of a draft tree verified in one launch (gfx950).
//
// Tree mode of the verify forward (lucebox-hub internal.h, QwenGraphInputs::parent_ids; the
// capture is sized for 1 + tree budget positions in create_target_cache).  Node i hangs off
// parent[i] (-1: the committed state); its state is its parent's state advanced by node i's
// token and its conv window runs along its root path, filled from the slot's conv state above the
// root.  Every node's state and 3-row conv state are captured so that gdn_rollback can commit any
// accepted node; the committed state and conv state are left untouched.
//
// One workgroup per (batch entry, value head).  A launch covers up to kTreeMaxNodes nodes (what one
// workgroup's LDS holds); a larger tree is consecutive launches over consecutive node ranges.  A node
// whose parent belongs to an earlier launch starts from that parent's captured state, which each
// lane reads back from exactly the capture elements it stored itself (the launch boundary orders
// the two), and its conv window reads the raw rows of ancestors outside the launch from qkv.
// A prologue stages the raw q|k|v rows of the launch's nodes in LDS (global_load_lds), computes
// every node's conv output, gate and beta into LDS, and builds a depth-first processing schedule.  The node loop then runs in DFS order: a node whose
// parent is the node just processed continues from the state in registers (each step is
// Geo::step, the same arithmetic as the chain kernel).  A node with two or more children leaves a
// register copy of its state in one of kTreeSaved save slots, which its later children restore;
// children are visited lightest subtree first, so a slot is released (its node's last child
// started) before the deepest descent, and few slots cover a whole tree.  When a parent's copy was
// evicted, its root path is re-run from the nearest saved ancestor or the committed state
// (compute only, nothing stored).  No state is ever re-read from memory, so the loop never waits
// on the memory counter that the capture stores occupy.
#include "gdn_device.h"
#include "gdn_geo.h"
#include "gdn_internal.h"

#include <type_traits>

namespace gdn {

constexpr int kTreeMaxNodes = 64;      // nodes per launch
constexpr int kTreeMaxTotal = 1024;    // nodes per call
constexpr int kTreeSaved = 3;  // register save slots for states that later siblings restore
// Schedule entry: node index within the launch (bits 0-7) | restart-from-committed-state flag |
// capture-and-output flag | 1 + the save slot restored before the step (bits 10-11, 0: none) |
// 1 + the save slot written after it (bits 12-13, 0: none) | start-from-the-parent's-capture flag
// (the parent belongs to an earlier launch).
constexpr int kSchedRestart = 0x100;
constexpr int kSchedEmit = 0x200;
constexpr int kSchedRestoreShift = 10;
constexpr int kSchedSaveShift = 12;
constexpr int kSchedLoad = 0x4000;
constexpr int kSchedMax = kTreeMaxNodes * (kTreeMaxNodes + 1) / 2 + kTreeMaxNodes;

// Waves per head: twice the chain kernel's.  A tree's node steps form one dependent chain per
// (slot, head) (64 nodes plus the root-path recomputations of DFS restarts), so the step latency,
// not bytes, bounds the kernel; spreading the state's rows over more waves halves each lane's work
// per step.  Each lane still holds whole 16-lane column groups, so the per-row sums, and the
// results, are the same bits as in the chain kernel.
template <int D>
struct TreeWaves {
    static constexpr int value = 2 * WavesPerHead<D>::value;
};

template <int D, typename act_t>
struct TreeLds {
    __host__ __device__ static size_t raw_bytes(int T) { return (size_t)T * 3 * D * sizeof(act_t); }
    __host__ __device__ static size_t o_bytes(int T) { return (size_t)T * D * sizeof(float); }
    __host__ __device__ static size_t region(int T)
    {
        const size_t r = raw_bytes(T) > o_bytes(T) ? raw_bytes(T) : o_bytes(T);
        return (r + 15) & ~(size_t)15;
    }
    __host__ __device__ static size_t total(int T)
    {
        return sizeof(float) * 3 * (size_t)T * D         // qs, ks, vs
               + region(T)                                // raw rows, then os
               + sizeof(float) * 4 * (size_t)T            // rho, beta, k.q
               + sizeof(int) * 4 * (size_t)T              // ancestors 1..3 (+ pad)
               + sizeof(uint16_t) * kSchedMax + 16;       // schedule + its length
    }
};

// Depth-first schedule of a tree of T <= 64 nodes, built by one wave with lane n standing for node
// n and every step a whole-wave one (cross-lane reads, no LDS round trips, no sequential walk over
// the nodes).  Siblings (roots too) are visited in order of subtree size, then index, so that the
// largest subtree comes last.  Save slots: a node with two or more children leaves a copy of its
// state for its later children in slot d mod kTreeSaved, where d counts its ancestors still
// awaiting a later child when it is visited (the nodes whose copies are live at that moment, each
// in its own slot d' mod kTreeSaved); a later child restores the parent's copy unless a node
// visited in between was saved at depth d' >= d + kTreeSaved, which overwrote it, and then re-runs
// the parent's root path from the committed state instead (compute only, nothing stored).
// anc[4 n + 3] holds node n's parent (a node index of the whole call); the launch's nodes start at
// base.  A node whose parent lies before base is a root of the launch that starts from the parent's
// capture instead of the committed state.
__device__ __forceinline__ void build_schedule(int T, int base, int lane, const int *anc, uint16_t *sched, int *nsched)
{
    auto rl = [](int v, int l) { return __builtin_amdgcn_readlane(v, l); };  // v of lane l (uniform l)
    auto from = [](int v, int l) { return __shfl(v, l); };                   // v of lane l (per lane)
    const bool node = lane < T;
    int par = -1;
    bool ext = false;  // the node's parent is in an earlier launch
    if (node) {
        const int p = anc[lane * 4 + 3];
        const int pg = (p >= -1 && p < base + lane) ? p : -1;  // a malformed parent makes a root
        par = pg >= base ? pg - base : -1;
        ext = pg >= 0 && pg < base;
    }
    // ancestor-or-self mask (two words) and depth: walk up, one level per round
    uint32_t am_lo = node && lane < 32 ? 1u << lane : 0u, am_hi = node && lane >= 32 ? 1u << (lane - 32) : 0u;
    // The loops below are branch-free (selects, not conditions) and the ones over all lanes run a
    // fixed 64 times, lanes past T standing for no node (parent -1, size 0, no ancestors): they add
    // nothing, and the loops unroll.
    int depth = 0, root = lane;  // root: the topmost ancestor within the launch
    for (int a = par; __any(a >= 0);) {
        const bool in = a >= 0;
        const int up = from(par, in ? a : 0);
        am_lo |= in && a < 32 ? 1u << (a & 31) : 0u;
        am_hi |= in && a >= 32 ? 1u << (a & 31) : 0u;
        depth += in ? 1 : 0;
        root = in ? a : root;
        a = in ? up : -1;
    }
    const bool root_ext = from((int)ext, root) != 0;  // a re-run of the root path starts from a capture
    // children and subtree sizes
    int kids = 0, size = 0;
#pragma unroll
    for (int m = 0; m < 64; ++m) {
        const int pm = rl(par, m);
        const uint32_t lo = (uint32_t)rl((int)am_lo, m), hi = (uint32_t)rl((int)am_hi, m);
        kids += pm == lane ? 1 : 0;
        size += (int)(((lane < 32 ? lo : hi) >> (lane & 31)) & 1u);
    }
    // sizes of the siblings visited before this node
    int off = 0;
#pragma unroll
    for (int m = 0; m < 64; ++m) {
        const int pm = rl(par, m), sm = rl(size, m);
        const bool before = (pm == par) & ((sm < size) | ((sm == size) & (m < lane)));
        off += before ? sm : 0;
    }
    // preorder position and d: walk up again, summing each level's offset and whether it keeps its
    // parent awaiting a later child
    // (every cross-lane read below runs on the whole wave, outside any condition: a lane reads
    // only lanes that execute the read with it)
    const int pp = par < 0 ? 0 : par;
    const int pkids = from(kids, pp), psize = from(size, pp);
    const int opens = (par >= 0 && pkids >= 2 && off + size != psize - 1) ? 1 : 0;
    const int step = off + (par >= 0 ? 1 : 0);
    int pre = 0, d = 0;
    for (int c = node ? lane : -1; __any(c >= 0);) {
        const bool in = c >= 0;
        const int cc = in ? c : 0;
        const int sp = from(step, cc), op = from(opens, cc), pc = from(par, cc);
        pre += in ? sp : 0;
        d += in ? op : 0;
        c = in ? pc : -1;
    }
    if (!node) pre = lane;  // the lanes past T keep their places: pre is a permutation of the lanes
    const int ord = __builtin_amdgcn_ds_permute(pre * 4, lane);  // ord[i]: the node at position i
    const int prev = from(ord, pre > 0 ? pre - 1 : 0);
    const bool restore = node && par >= 0 && pre > 0 && par != prev;
    const int dq = from(d, pp), preq = from(pre, pp), depq = from(depth, pp);
    const uint32_t amq_lo = (uint32_t)from((int)am_lo, pp), amq_hi = (uint32_t)from((int)am_hi, pp);
    // the deepest save between the parent's visit and this one
    const int dsave = node && kids >= 2 ? d : -1;
    const int dsave_at = from(dsave, ord);  // by position
    int dmax = -1;
#pragma unroll
    for (int i = 0; i < 64; ++i) {  // positions past T hold no node: dsave -1
        const int v = rl(dsave_at, i);
        dmax = ((i > preq) & (i < pre) & (v > dmax)) ? v : dmax;
    }
    const bool live = dmax < dq + kTreeSaved;
    const bool rerun = restore && !live;
    // entries: the re-run root path (root .. parent), then the node; offsets by position
    const int cnt = node ? 1 + (rerun ? depq + 1 : 0) : 0;
    const int cnt_ord = from(cnt, ord);
    const int cnt_at = lane < T ? cnt_ord : 0;
    int incl = cnt_at;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o);
        if (lane >= o) incl += y;
    }
    const int first = from(incl - cnt_at, pre);  // this node's first schedule entry
    if (node) {
        int e = lane | kSchedEmit;
        if (par < 0)
            e |= ext ? kSchedLoad : kSchedRestart;
        else if (restore && live)
            e |= (dq % kTreeSaved + 1) << kSchedRestoreShift;
        if (kids >= 2) e |= (d % kTreeSaved + 1) << kSchedSaveShift;
        int at = first;
        if (rerun) {  // the parent's root path in index order: ancestors have smaller indices
            uint32_t lo = amq_lo, hi = amq_hi;
            for (int k = 0; lo | hi; ++k) {
                const int x = lo ? __builtin_ctz(lo) : 32 + __builtin_ctz(hi);
                if (lo)
                    lo &= lo - 1;
                else
                    hi &= hi - 1;
                sched[at++] = (uint16_t)(x | (k == 0 ? (root_ext ? kSchedLoad : kSchedRestart) : 0));
            }
        }
        sched[at] = (uint16_t)e;
    }
    const int total = rl(incl, 63);
    if (lane == 0) *nsched = total;
}

// LATER: the launch follows an earlier one of the same call (its first node is not node 0); only
// such launches carry the code that reads state and conv rows written or staged before them.
template <int D, bool ACT_BF16, bool OUT_BF16, bool QKN, bool LATER>
__global__ __launch_bounds__(TreeWaves<D>::value * 64) void verify_tree_kernel(VerifyArgs a)
{
    using act_t = typename std::conditional<ACT_BF16, uint16_t, float>::type;
    using L = TreeLds<D, act_t>;
    constexpr int NW = TreeWaves<D>::value;
    using G = Geo<D, NW>;
    constexpr int VEC = 16 / (int)sizeof(act_t);
    constexpr int NCH = 3 * D;  // q | k | v channels of this value head
    const int R = a.n_vh / a.n_kh;
    const int T = a.T;      // nodes of the whole call: the row stride of qkv, z, alpha, beta, parent, out
    const int base = LATER ? a.t0 : 0;  // first node of this launch
    const int NT = a.nt;    // nodes of this launch, 1 .. kTreeMaxNodes
    const int tid = threadIdx.x;
    const int nthr = NW * 64;
    const int wave = tid >> 6, lane = tid & 63;
    const int rg = lane >> 4, cg = lane & 15;

    const int b = blockIdx.x / a.n_vh;
    const int h = blockIdx.x % a.n_vh;
    const int hk = h / R;
    const bool lead = (h % R) == 0;  // writes the shared q / k channels of the conv capture
    const int s = a.slot_ids[b];
    if (s < 0 || s >= a.n_pool) return;  // uniform over the workgroup

    extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
    // LDS rows are the launch's nodes, 0 .. NT-1 (node base + i of the call)
    float *qs = reinterpret_cast<float *>(smem_raw);  // [NT][D]
    float *ks = qs + NT * D;                           // [NT][D]
    float *vs = ks + NT * D;                           // [NT][D]   rows in perm order
    act_t *raw = reinterpret_cast<act_t *>(vs + NT * D);  // [NT][3D]  raw q|k|v rows (prologue)
    float *os = reinterpret_cast<float *>(raw);           // [NT][D]   readout, rows in perm order (loop)
    float *rbk = reinterpret_cast<float *>(reinterpret_cast<unsigned char *>(raw) + L::region(NT));  // [NT][4]
    // [NT][4]: ancestors 1..3 (>= 0 node of the call, -1-r conv row r), parent (node of the call)
    int *anc = reinterpret_cast<int *>(rbk + 4 * NT);
    uint16_t *sched = reinterpret_cast<uint16_t *>(anc + 4 * NT);
    int *nsched = reinterpret_cast<int *>(sched + kSchedMax);

    const int C = a.C;
    const int q0 = hk * D, k0 = a.n_kh * D + hk * D, v0 = 2 * a.n_kh * D + h * D;
    const float *cs_s = a.conv_state + (size_t)s * 3 * C;
    const int32_t *par = a.parent + (size_t)b * T;
    const act_t *qkv_b = static_cast<const act_t *>(a.qkv) + (size_t)b * T * C;
    auto gchan = [&](int lc) -> int { return lc < D ? q0 + lc : (lc < 2 * D ? k0 + (lc - D) : v0 + (lc - 2 * D)); };
    auto to_f32 = [](act_t x) -> float {
        if constexpr (ACT_BF16)
            return bf16_to_f32(x);
        else
            return x;
    };
    // a malformed parent (outside [-1, n)) is treated as -1: the node starts from the committed state.
    // Parents of the launch's nodes are read from LDS (slot 3 of each node's ancestor record, filled
    // once at staging), those of earlier nodes from the parent array.
    auto parent_of = [&](int n) -> int {  // n: node of the call
        const int p = (!LATER || n >= base) ? anc[(n - base) * 4 + 3] : par[n];
        return (p >= -1 && p < n) ? p : -1;
    };

    // ================= stage: raw rows of all nodes into LDS, everything else into registers ====
    const int nvr = NCH / VEC;
    for (int it = tid; it < NT * nvr; it += nthr) {
        const int r = it / nvr, lc = (it % nvr) * VEC;
        lds_dma16(qkv_b + (uint32_t)((base + r) * C + gchan(lc)), raw + it * VEC);
    }
    // conv channels: thread 64 + lc takes channel lc (wave 0 builds the schedule meanwhile)
    static_assert(NCH <= 64 * (NW - 1) && NCH % 64 == 0, "one conv channel per thread of whole waves 1 ..");
    const int lc = tid - 64;
    const bool conv_thread = lc >= 0 && lc < NCH;
    f4 wv = {0.f, 0.f, 0.f, 0.f};
    float cs0 = 0.f, cs1 = 0.f, cs2 = 0.f;  // the slot's conv state rows
    if (conv_thread) {
        const int gc = gchan(lc);
        wv = *reinterpret_cast<const f4 *>(a.conv_w + (size_t)gc * 4);
        cs0 = cs_s[(uint32_t)gc];
        cs1 = cs_s[(uint32_t)(C + gc)];
        cs2 = cs_s[(uint32_t)(2 * C + gc)];
    }
    // alpha, beta and the parent of node base + tid.  The loads sit outside any branch (threads past
    // the launch's nodes load its last node's) and nothing is computed from them before the wait
    // below: a bf16 conversion, or a branch join over a loaded register, would make the compiler wait
    // for every load issued so far before the state loads start.
    using word_t = typename std::conditional<ACT_BF16, uint16_t, uint32_t>::type;  // bf16 or fp32 bits
    const int node = base + min(tid, NT - 1);
    const size_t tok = ((size_t)b * T + node) * a.n_vh + h;
    uint32_t al_raw = static_cast<const word_t *>(a.alpha)[tok];
    uint32_t be_raw = static_cast<const word_t *>(a.beta)[tok];
    int par_raw = par[node];
    float alog = a.A_log[h], dtb = a.dt_bias[h];
    // the committed state: kept in registers for the whole launch (restart point)
    float R0[G::RPL][G::CPL];
    const int wih = wave;
    const int row0 = wih * G::RPW + rg;
    const float *st_ptr = a.state + ((size_t)s * a.n_vh + h) * (size_t)D * D + (size_t)row0 * D + cg * 4;
#pragma unroll
    for (int i = 0; i < G::RPL; ++i)
#pragma unroll
        for (int c4 = 0; c4 < G::NC4; ++c4) {
            const f4 v = *reinterpret_cast<const f4 *>(st_ptr + (size_t)(4 * i) * D + 64 * c4);
#pragma unroll
            for (int e = 0; e < 4; ++e) R0[i][4 * c4 + e] = v[e];
        }
    // z of the nodes this thread's 16-lane group normalises in the epilogue, loaded now: loaded
    // after the node loop, it would wait behind the whole capture stream on the one memory counter
    constexpr int EPL = D / 16;                         // z elements per lane and node
    constexpr int NGRP = NW * 4;                        // 16-lane groups
    constexpr int NPG = (kTreeMaxNodes + NGRP - 1) / NGRP;  // nodes per group
    word_t zr[NPG][EPL];
#pragma unroll
    for (int k = 0; k < NPG; ++k) {
        const int zn = base + min((tid >> 4) + k * NGRP, NT - 1);  // past the last node: a valid row, unused
        const word_t *zp = static_cast<const word_t *>(a.z) + (((size_t)b * T + zn) * a.n_vh + h) * D + cg * EPL;
#pragma unroll
        for (int e = 0; e < EPL; ++e) zr[k][e] = zp[e];
    }
    float nwr[EPL];  // the norm weights of this lane's columns, for the same reason
#pragma unroll
    for (int e = 0; e < EPL; ++e) nwr[e] = a.norm_w[cg * EPL + e];
    __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0): raw rows landed, registers loaded
    asm volatile("" : "+v"(al_raw), "+v"(be_raw), "+v"(par_raw), "+v"(alog), "+v"(dtb));  // nothing above
    auto word_f32 = [](uint32_t w) -> float {
        if constexpr (ACT_BF16)
            return bf16_to_f32((uint16_t)w);
        else
            return __builtin_bit_cast(float, w);
    };
    if (tid < NT) {
        const float g = -expf(alog) * softplus_f(word_f32(al_raw) + dtb);
        rbk[tid * 4 + 0] = expf(g);
        rbk[tid * 4 + 1] = word_f32(be_raw);
        anc[tid * 4 + 3] = par_raw;
    }
    __syncthreads();
    // ancestors 1..3 of every node (its conv window); where the root path ends, the slot's conv
    // state rows fill in: with L path nodes inside the window, ancestor j > L-1 is conv row 2-(j-L)
    if (tid < NT) {
        int code[3];
        int m = base + tid, L = 1;
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            m = m >= 0 ? parent_of(m) : -1;
            code[k] = m;
            L += m >= 0 ? 1 : 0;
        }
#pragma unroll
        for (int k = 0; k < 3; ++k)
            if (code[k] < 0) code[k] = -1 - (2 - (k + 1 - L));  // -1 - conv row
        anc[tid * 4 + 0] = code[0];
        anc[tid * 4 + 1] = code[1];
        anc[tid * 4 + 2] = code[2];
    }
    __syncthreads();

    if (wave == 0) {
        build_schedule(NT, base, lane, anc, sched, nsched);
    } else if (conv_thread) {
        // ================= conv of every node (one thread per channel) + conv-state capture =====
        float *cct = a.cap_conv + ((size_t)s * a.t_cap + base) * 3 * C;  // [t_cap][3][C] of this slot, from node base
        const int gc = gchan(lc);
        const bool own = lc >= 2 * D || lead;
        float *dst = lc < D ? qs + lc : (lc < 2 * D ? ks + (lc - D) : vs + G::perm(lc - 2 * D));
        // the row an ancestor code names; the conv-state rows come in as values, not captures: a
        // select between captured variables becomes a load through a select of their addresses,
        // which keeps them in scratch memory
        // (the row is read unconditionally, the launch's first node's for a code outside the launch,
        // so that no read sits under a branch and a batch's reads are all in flight together; a node
        // of an earlier launch is read from qkv, in launches after the first)
        auto X = [raw, lc, gc, base, qkv_b, C, to_f32](int code, float c0, float c1, float c2) -> float {
            const float h = code == -1 ? c0 : (code == -2 ? c1 : c2);
            const float r = to_f32(raw[max(code - base, 0) * NCH + lc]);
            if constexpr (LATER) {
                const float e = to_f32(qkv_b[(size_t)min(max(code, 0), base - 1) * C + gc]);
                return code >= base ? r : (code >= 0 ? e : h);
            } else {
                return code >= 0 ? r : h;
            }
        };
        // Nodes in batches of CB = 16: one LDS read brings the batch's ancestor codes, lane 4 j + i
        // holding code i of node n0 + j, and they are taken from there lane by lane (readlane: the
        // conv waves are whole); then every row read of the batch is issued before its first store
        // (the compiler cannot move a read above a store to LDS it may alias).
        constexpr int CB = 16;
#pragma unroll 1
        for (int n0 = 0; n0 < NT; n0 += CB) {
            const int codes = anc[min(n0 + (lane >> 2), NT - 1) * 4 + (lane & 3)];
            float x[CB][4];
            // Past the first levels of a tree every ancestor of a batch's nodes is staged in this
            // launch: then the rows are read straight, without X's selects (the same values).
            if (__all((lane & 3) == 3 || codes >= base)) {
#pragma unroll
                for (int j = 0; j < CB; ++j) {
                    const int n = min(n0 + j, NT - 1);
#pragma unroll
                    for (int i = 0; i < 3; ++i)
                        x[j][i] = to_f32(raw[(__builtin_amdgcn_readlane(codes, 4 * j + 2 - i) - base) * NCH + lc]);
                    x[j][3] = to_f32(raw[n * NCH + lc]);
                }
            } else {
#pragma unroll
                for (int j = 0; j < CB; ++j) {
                    const int n = min(n0 + j, NT - 1);
                    x[j][0] = X(__builtin_amdgcn_readlane(codes, 4 * j + 2), cs0, cs1, cs2);
                    x[j][1] = X(__builtin_amdgcn_readlane(codes, 4 * j + 1), cs0, cs1, cs2);
                    x[j][2] = X(__builtin_amdgcn_readlane(codes, 4 * j), cs0, cs1, cs2);
                    x[j][3] = to_f32(raw[n * NCH + lc]);
                }
            }
#pragma unroll
            for (int j = 0; j < CB; ++j) {
                const int n = n0 + j;
                if (n >= NT) break;
                float y = conv4(wv, x[j][0], x[j][1], x[j][2], x[j][3]);
                if constexpr (QKN) y = y * sigmoid_f(y);
                dst[n * D] = y;
                if (own) {  // 3-row conv state after node n: [ancestor 2, ancestor 1, n], non-temporal
                    float *cp = cct + (size_t)n * 3 * C + gc;
                    __builtin_nontemporal_store(x[j][1], cp);
                    __builtin_nontemporal_store(x[j][2], cp + (size_t)C);
                    __builtin_nontemporal_store(x[j][3], cp + (size_t)2 * C);
                }
            }
        }
    }
    __syncthreads();
    // ================= the node loop in schedule order =================
    float S[G::RPL][G::CPL];
#pragma unroll
    for (int i = 0; i < G::RPL; ++i)
#pragma unroll
        for (int c = 0; c < G::CPL; ++c) S[i][c] = R0[i][c];
    const size_t hd = (size_t)D * D;
    float *cap_base = a.cap_ssm + ((size_t)s * a.t_cap * a.n_vh + h) * hd + (size_t)row0 * D + cg * 4;  // node 0
    const size_t cap_nstride = (size_t)a.n_vh * hd;
    float SV[kTreeSaved][G::RPL][G::CPL];  // save slots (indexed by constants only: registers)
    auto copy_state = [](float (&dst)[G::RPL][G::CPL], const float (&src)[G::RPL][G::CPL]) {
#pragma unroll
        for (int i = 0; i < G::RPL; ++i)
#pragma unroll
            for (int c = 0; c < G::CPL; ++c) dst[i][c] = src[i][c];
    };
    const int ns = *nsched;
#pragma unroll 1
    for (int k = 0; k < ns; ++k) {
        const int e = __builtin_amdgcn_readfirstlane(sched[k]);  // uniform: scalar branches below
        const int n = e & 0xff;
        const int rs = (e >> kSchedRestoreShift) & 3, sv = (e >> kSchedSaveShift) & 3;
        if (e & kSchedRestart) copy_state(S, R0);
        if (LATER && (e & kSchedLoad)) {  // the parent's state, from the capture an earlier launch wrote
            const float *src = cap_base + (size_t)anc[n * 4 + 3] * cap_nstride;
#pragma unroll
            for (int i = 0; i < G::RPL; ++i)
#pragma unroll
                for (int c4 = 0; c4 < G::NC4; ++c4) {
                    const f4 v = *reinterpret_cast<const f4 *>(src + (size_t)(4 * i) * D + 64 * c4);
#pragma unroll
                    for (int e4 = 0; e4 < 4; ++e4) S[i][4 * c4 + e4] = v[e4];
                }
        }
#pragma unroll
        for (int j = 0; j < kTreeSaved; ++j)
            if (rs == j + 1) copy_state(S, SV[j]);
        const f4 sc = *reinterpret_cast<const f4 *>(rbk + n * 4);
        float o[G::RPL];
        G::template step<QKN>(S, ks + n * D, qs + n * D, vs + n * D + wih * G::RPW + rg * G::RPL, sc[0], sc[1], cg, o);
        if (e & kSchedEmit) {
            if (cg == 0) {
                float *od = os + n * D + wih * G::RPW + rg * G::RPL;
#pragma unroll
                for (int i = 0; i < G::RPL; ++i) od[i] = o[i];
            }
            float *cp = cap_base + (size_t)(base + n) * cap_nstride;
#pragma unroll
            for (int i = 0; i < G::RPL; ++i)
#pragma unroll
                for (int c4 = 0; c4 < G::NC4; ++c4) {
                    const f4 v = {S[i][4 * c4], S[i][4 * c4 + 1], S[i][4 * c4 + 2], S[i][4 * c4 + 3]};
                    store_stream(cp + (size_t)(4 * i) * D + 64 * c4, v);
                }
        }
#pragma unroll
        for (int j = 0; j < kTreeSaved; ++j)
            if (sv == j + 1) copy_state(SV[j], S);
    }
    __syncthreads();

    // ================= epilogue: out = o / sqrt(mean(o^2) + eps) * norm_w * silu(z) =================
    const int grp = tid >> 4;
#pragma unroll
    for (int k = 0; k < NPG; ++k) {
        const int n = grp + k * NGRP;
        if (n >= NT) break;  // uniform over the 16-lane group
        const float *osrc = os + n * D;
        float ov[EPL];
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            ov[e] = osrc[G::perm(cg * EPL + e)];
            ss += ov[e] * ov[e];
        }
        ss = row16_sum(ss);
        const float inv = 1.0f / sqrtf(ss / (float)D + a.eps);
        const size_t ob = (((size_t)b * T + base + n) * a.n_vh + h) * D + cg * EPL;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            const float zz = word_f32(zr[k][e]);
            const float y = ov[e] * inv * nwr[e] * (zz * sigmoid_f(zz));
            if constexpr (OUT_BF16)
                static_cast<uint16_t *>(a.out)[ob + e] = f32_to_bf16(y);
            else
                static_cast<float *>(a.out)[ob + e] = y;
        }
    }
}

size_t verify_tree_lds_bytes(int d, int T, bool act_bf16)
{
    if (T < 1 || T > kTreeMaxTotal) return (size_t)-1;
    T = T < kTreeMaxNodes ? T : kTreeMaxNodes;  // one launch's nodes
    if (d == 128) return act_bf16 ? TreeLds<128, uint16_t>::total(T) : TreeLds<128, float>::total(T);
    return act_bf16 ? TreeLds<64, uint16_t>::total(T) : TreeLds<64, float>::total(T);
}

// Consecutive launches over consecutive ranges of at most kTreeMaxNodes nodes, on one stream: a
// launch reads the captures of earlier ranges only after their launches have finished.
template <int D, bool AB, bool OB, bool QKN>
static hipError_t launch_tree_t(const VerifyArgs &a0, hipStream_t stream)
{
    for (int t0 = 0; t0 < a0.T; t0 += kTreeMaxNodes) {
        VerifyArgs a = a0;
        a.t0 = t0;
        a.nt = a0.T - t0 < kTreeMaxNodes ? a0.T - t0 : kTreeMaxNodes;
        const size_t lds = verify_tree_lds_bytes(D, a.nt, AB);
        if (t0 == 0)
            hipLaunchKernelGGL((verify_tree_kernel<D, AB, OB, QKN, false>), dim3(a.n_batch * a.n_vh),
                               dim3(TreeWaves<D>::value * 64), lds, stream, a);
        else
            hipLaunchKernelGGL((verify_tree_kernel<D, AB, OB, QKN, true>), dim3(a.n_batch * a.n_vh),
                               dim3(TreeWaves<D>::value * 64), lds, stream, a);
        if (hipError_t e = hipGetLastError()) return e;
    }
    return hipSuccess;
}
template <int D, bool AB, bool OB>
static hipError_t launch_tree_q(const VerifyArgs &a, const LaunchCfg &c, hipStream_t s)
{
    return c.qk_norm ? launch_tree_t<D, AB, OB, true>(a, s) : launch_tree_t<D, AB, OB, false>(a, s);
}
template <int D, bool AB>
static hipError_t launch_tree_o(const VerifyArgs &a, const LaunchCfg &c, hipStream_t s)
{
    return c.out_bf16 ? launch_tree_q<D, AB, true>(a, c, s) : launch_tree_q<D, AB, false>(a, c, s);
}
template <int D>
static hipError_t launch_tree_a(const VerifyArgs &a, const LaunchCfg &c, hipStream_t s)
{
    return c.act_bf16 ? launch_tree_o<D, true>(a, c, s) : launch_tree_o<D, false>(a, c, s);
}

hipError_t launch_verify_tree(const VerifyArgs &a, const LaunchCfg &c, hipStream_t stream)
{
    if (a.d == 128) return launch_tree_a<128>(a, c, stream);
    if (a.d == 64) return launch_tree_a<64>(a, c, stream);
    return hipErrorInvalidValue;
}

}  // namespace gdn
