// gdn_linear.hip - the GDN block's projections, y = x W^T, on MFMA (gfx950).
//
// lucebox-hub internal.h, struct TargetLayer: the block reads its activations through the fused
// q / k / v projection (wqkv), the z projection (wqkv_gate) and the per-token beta and alpha
// projections (ssm_beta, ssm_alpha), and writes its result through ssm_out.  Each is a product of
// the token rows x [M][K] (bf16) with a weight W [N][K] (bf16, one output feature per row, input
// index fastest), accumulated in fp32.  One launch may feed several destinations: the product's
// columns are split into segments, each with its own pointer, row stride, storage type and an
// optional sigmoid (beta is sigmoid(x W_beta^T)), so the four input projections are one GEMM over
// the concatenated weight.
//
// Tiling: a workgroup computes a block of y with a grid of waves, each a grid of 16 x 16 tiles of
// v_mfma_f32_16x16x32_bf16 (256 x 256 or 128 x 128 blocks for many rows, 16 x 16 to 32 x 64 for
// few).  K advances 64 at a time, one barrier per step: the next x and W tiles travel into a
// buffer of the LDS (two, or four for few rows) by global_load_lds while the current ones are
// multiplied.  Within an
// LDS tile row (64 bf16 = 8 chunks of 16 bytes) chunk c of row r sits at position c ^ (r & 7),
// so the 16 rows an operand load touches spread over the banks; the DMA writes LDS linearly, so
// the swizzle is applied by choosing the global chunk each lane fetches.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

constexpr int kLBK = 64;  // k depth of a tile

// s_waitcnt immediate: at most n vector-memory operations outstanding (vmcnt bits 3:0 and 15:14;
// expcnt and lgkmcnt left at their maxima).
constexpr int vmcnt_imm(int n) { return 0x0F70 | (n & 0xF) | ((n >> 4) << 14); }
constexpr int kLChunks = kLBK / 8;  // 16-byte chunks per tile row

__device__ __forceinline__ f4 mfma_bf16(bf16x8_t a, bf16x8_t b, f4 c)
{
#if defined(__HIP_DEVICE_COMPILE__)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
#else
    (void)a;
    (void)b;
    return c;
#endif
}

// Scheduling groups (__builtin_amdgcn_sched_group_barrier): n instructions of one kind, groups
// placed in the order of the calls within the enclosing block.
constexpr int kSchedMfma = 0x008, kSchedDsRead = 0x100;
#define sched_group(mask, n) __builtin_amdgcn_sched_group_barrier((mask), (n), 0)

// LDS byte offset of chunk c of tile row r
__device__ __forceinline__ int lchunk(int r, int c) { return (r * kLChunks + (c ^ (r & 7))) * 16; }

// Workgroup tile (16 WM GM) x (16 WN GN): GM x GN waves, each (16 WM) x (16 WN) = WM x WN MFMA
// tiles.
template <int GM, int GN, int WM, int WN, int NBUF = 2>
struct LinTile {
    static constexpr int THREADS = 64 * GM * GN;
    static constexpr int BM = 16 * WM * GM, BN = 16 * WN * GN;
    // x and W transfers per thread and k tile (at most: with XE / WE false the last round of
    // transfers covers only the first threads, whole waves)
    static constexpr int XT = (BM * kLChunks + THREADS - 1) / THREADS;
    static constexpr int WT = (BN * kLChunks + THREADS - 1) / THREADS;
    static constexpr bool XE = BM * kLChunks % THREADS == 0, WE = BN * kLChunks % THREADS == 0;
    static constexpr size_t lds = NBUF * (size_t)(BM + BN) * kLBK * 2;  // NBUF buffers of x and W tiles
    static_assert(XT >= 1 && WT >= 1 && (NBUF - 1) * (XT + WT) < 64, "tile transfer counts");
    static_assert((BM * kLChunks % THREADS) % 64 == 0 && (BN * kLChunks % THREADS) % 64 == 0,
                  "a partial round of transfers covers whole waves");
    // with more than two buffers the wait for a k tile counts this thread's later transfers, which
    // must then be the same for every thread
    static_assert(NBUF == 2 || (XE && WE), "uneven transfer counts need two buffers");
};

// Wait until at most `later` k tiles of TPT transfers each are in flight (s_waitcnt takes an
// immediate, so one instruction per count; later <= MAXL).
template <int TPT, int MAXL>
__device__ __forceinline__ void wait_tiles(int later)
{
    static_assert(MAXL <= 6 && MAXL * TPT < 64, "vmcnt range");
    switch (MAXL > 0 ? later : 0) {
    case 6: __builtin_amdgcn_s_waitcnt(vmcnt_imm(6 * TPT)); break;
    case 5: __builtin_amdgcn_s_waitcnt(vmcnt_imm(5 * TPT)); break;
    case 4: __builtin_amdgcn_s_waitcnt(vmcnt_imm(4 * TPT)); break;
    case 3: __builtin_amdgcn_s_waitcnt(vmcnt_imm(3 * TPT)); break;
    case 2: __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * TPT)); break;
    case 1: __builtin_amdgcn_s_waitcnt(vmcnt_imm(TPT)); break;
    default: __builtin_amdgcn_s_waitcnt(vmcnt_imm(0)); break;
    }
}

// NBUF k tiles are buffered: NBUF - 1 of them travel while one is multiplied.
template <int GM, int GN, int WM, int WN, int NBUF>
__global__ __launch_bounds__(64 * GM * GN) void linear_kernel(LinearArgs a)
{
    using TL = LinTile<GM, GN, WM, WN, NBUF>;
    constexpr int BM = TL::BM, BN = TL::BN, kLThreads = TL::THREADS;
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];  // [buffer][x tile | W tile]
    constexpr int XB = BM * kLBK * 2, BUF = (BM + BN) * kLBK * 2;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int li = lane & 15, lg = lane >> 4;
    const int wm = wave / GN, wn = wave % GN;  // the wave's place in the GM x GN grid
    // Tiles are numbered n-major, m fastest (t = n_tile * mt + m_tile), and workgroups are dealt
    // to the 8 XCDs in turn; XCD x takes a contiguous tile range (the first T mod 8 XCDs one tile
    // more than the others), so the workgroups sharing a weight tile run on one XCD, one after
    // another, and read it from that XCD's L2 instead of once per XCD.
    const int mt = (a.M + BM - 1) / BM, ntiles = gridDim.x;
    const int xcd = blockIdx.x % 8, q8 = ntiles / 8, r8 = ntiles % 8;
    const int t = xcd * q8 + min(xcd, r8) + blockIdx.x / 8;
    const int m0 = (t % mt) * BM, n0 = (t / mt) * BN;
    const int K = a.K;

    // this thread's transfers of a k tile: LDS position p = tid + 256 i (row p / 8, slot p % 8)
    // holds chunk slot ^ (row & 7) of that row; rows past M or N re-read the last row (their
    // results are never stored), so every thread issues the same number of transfers
    const uint16_t *xsrc[TL::XT], *wsrc[TL::WT];
#pragma unroll
    for (int i = 0; i < TL::XT; ++i) {
        const int p = tid + kLThreads * i, r = p / kLChunks, c = (p % kLChunks) ^ (r & 7);
        xsrc[i] = a.x + (size_t)min(m0 + r, a.M - 1) * K + 8 * c;
    }
#pragma unroll
    for (int i = 0; i < TL::WT; ++i) {
        const int p = tid + kLThreads * i, r = p / kLChunks, c = (p % kLChunks) ^ (r & 7);
        wsrc[i] = a.w + (size_t)min(n0 + r, a.N - 1) * K + 8 * c;
    }
    auto issue = [&](int kt, int buf) {
        unsigned char *base = lds + buf * BUF;
#pragma unroll
        for (int i = 0; i < TL::XT; ++i)
            if (TL::XE || i < TL::XT - 1 || tid + kLThreads * i < BM * kLChunks)
                lds_dma16(xsrc[i] + kt * kLBK, base + (tid + kLThreads * i) * 16);
#pragma unroll
        for (int i = 0; i < TL::WT; ++i)
            if (TL::WE || i < TL::WT - 1 || tid + kLThreads * i < BN * kLChunks)
                lds_dma16(wsrc[i] + kt * kLBK, base + XB + (tid + kLThreads * i) * 16);
    };

    f4 acc[WM][WN];
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
        for (int j = 0; j < WN; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};

    const int nk = K / kLBK;
#pragma unroll
    for (int p = 0; p < NBUF - 1; ++p)
        if (p < nk) issue(p, p);
    constexpr int TPT = TL::XT + TL::WT;  // transfers per thread and k tile
#pragma unroll 1
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt % NBUF;
        // this thread's transfers of tile kt have landed; those of the (up to NBUF - 2) later tiles
        // already issued may travel
        wait_tiles<TPT, NBUF - 2>(min(nk - 1 - kt, NBUF - 2));
        // Every wave's transfers of tile kt have landed, and every wave is done with tile kt - 1,
        // so its buffer takes tile kt + NBUF - 1: one barrier per k tile.
        lds_barrier();
        if (kt + NBUF - 1 < nk) issue(kt + NBUF - 1, (kt + NBUF - 1) % NBUF);
        const unsigned char *xs = lds + buf * BUF, *ws = xs + XB;
        // every fragment of the tile's 32-deep steps is read before the first product, so the later
        // steps' reads are in flight while the earlier steps' products run
        constexpr int KS = kLBK / 32;
        bf16x8_t af[KS][WM], bf[KS][WN];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int c = 4 * ks + lg;  // this lane's chunk of the 32-deep step
#pragma unroll
            for (int i = 0; i < WM; ++i)
                af[ks][i] = *reinterpret_cast<const bf16x8_t *>(xs + lchunk(16 * WM * wm + 16 * i + li, c));
#pragma unroll
            for (int j = 0; j < WN; ++j)
                bf[ks][j] = *reinterpret_cast<const bf16x8_t *>(ws + lchunk(16 * WN * wn + 16 * j + li, c));
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int i = 0; i < WM; ++i)
#pragma unroll
                for (int j = 0; j < WN; ++j) acc[i][j] = mfma_bf16(af[ks][i], bf[ks][j], acc[i][j]);
        // Instruction order (the compiler would otherwise read each fragment just before its first
        // product and wait for it there): the first step's reads, then each later step's reads
        // spread between the previous step's products, so LDS latency hides behind MFMA work.
        constexpr int NR = WM + WN, NM = WM * WN, PER = NM / NR > 0 ? NM / NR : 1;
        sched_group(kSchedDsRead, NR);
#pragma unroll
        for (int ks = 1; ks < KS; ++ks) {
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                sched_group(kSchedMfma, PER);
                sched_group(kSchedDsRead, 1);
            }
            if (NM > PER * NR) sched_group(kSchedMfma, NM - PER * NR);
        }
        sched_group(kSchedMfma, NM);
    }

    // ---- epilogue: element (row 4 lg + r, column li) of each 16 x 16 tile to its segment
#pragma unroll
    for (int j = 0; j < WN; ++j) {
        const int n = n0 + 16 * WN * wn + 16 * j + li;
        if (n >= a.N) continue;
        int sgi = 0;
#pragma unroll
        for (int q = 1; q < kMaxLinearSegs; ++q)
            if (q < a.n_segs && n >= a.seg[q].n0) sgi = q;
        const LinearSeg &sg = a.seg[sgi];
        const int nc = n - sg.n0;
#pragma unroll
        for (int i = 0; i < WM; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + 16 * WM * wm + 16 * i + 4 * lg + r;
                if (m >= a.M) continue;
                float v = acc[i][j][r];
                if (sg.sigmoid) v = 1.0f / (1.0f + expf(-v));
                const size_t at = (size_t)m * sg.ld + nc;
                if (sg.bf16)
                    static_cast<uint16_t *>(sg.ptr)[at] = f32_to_bf16(v);
                else
                    static_cast<float *>(sg.ptr)[at] = v;
            }
    }
}

template <int GM, int GN, int WM, int WN, int NBUF = 2>
static hipError_t launch_tile(const LinearArgs &a, hipStream_t stream)
{
    using TL = LinTile<GM, GN, WM, WN, NBUF>;
    const unsigned tiles = (unsigned)((a.N + TL::BN - 1) / TL::BN) * (unsigned)((a.M + TL::BM - 1) / TL::BM);
    const dim3 grid(tiles);
    hipLaunchKernelGGL((linear_kernel<GM, GN, WM, WN, NBUF>), grid, dim3(TL::THREADS), TL::lds, stream, a);
    return hipGetLastError();
}

// Tile choice.  A k tile brings (BM + BN) x 64 operands into LDS for 2 BM BN x 64 flops, so larger
// workgroup tiles need fewer bytes per flop from L2, but a launch needs enough of them to spread
// over the 256 CUs, and smaller ones keep more k tiles in flight per CU.  The first of these whose
// tile count reaches its threshold is taken (thresholds measured on the GDN block's projections,
// 5120 -> 12352 and 4096 -> 5120, at 96 to 1024 rows):
//   256 x 256, 16 waves of 64 x 64, one workgroup per CU: >= 140 tiles (1024 rows of the
//     in-projection: 196 tiles, 134 us against 162 with 128 x 128; 768 rows: 129 against 146)
//   128 x 128, 16 waves of 32 x 32, two per CU: >= 280 (the out-projection at 1024 rows, 57 us)
//   64 x 128, 16 waves of 16 x 32: >= 280 (the in-projection at 192 - 256 rows, 52 - 55 us against
//     63 - 64 with 128 x 128)
//   64 x 64, 4 waves, three buffered k tiles: >= 280 (the out-projection at 256 - 384 rows, 30 us
//     against 48 with 128 x 128, which keeps one k tile in flight and waits on it at every step)
//   32 x 64, 4 waves, four buffered k tiles, otherwise (the out-projection up to 192 rows: 22 - 25
//     against 47 us).
// A few rows (one slot's drafted tokens) make the product a stream of the weight, read once:
// one-wave tiles of 16 (M <= 16) or 32 (M <= 32) rows by 16 columns spread it over N / 16
// workgroups with four buffered k tiles (16 x 5120 -> 12352: 20 us, 6.2 TB/s of weight, against
// 40 us with double-buffered 32 x 64 tiles; 16 x 4096 -> 5120: 14.5 against 31 us).
hipError_t launch_linear(const LinearArgs &a, hipStream_t stream)
{
    if (a.M <= 16) return launch_tile<1, 1, 1, 1, 4>(a, stream);
    if (a.M <= 32) return launch_tile<1, 1, 2, 1, 4>(a, stream);
    auto tiles = [&](int bm, int bn) { return (long)((a.M + bm - 1) / bm) * ((a.N + bn - 1) / bn); };
    if (a.M > 64) {
        if (tiles(256, 256) >= 140) return launch_tile<4, 4, 4, 4>(a, stream);
        if (tiles(128, 128) >= 280) return launch_tile<4, 4, 2, 2>(a, stream);
        if (tiles(64, 128) >= 280) return launch_tile<4, 4, 1, 2>(a, stream);
        if (tiles(64, 64) >= 280) return launch_tile<2, 2, 2, 2, 3>(a, stream);
    }
    return launch_tile<2, 2, 1, 2, 4>(a, stream);
}

}  // namespace gdn
