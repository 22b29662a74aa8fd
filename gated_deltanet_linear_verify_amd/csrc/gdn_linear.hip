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
// v_mfma_f32_16x16x32_bf16 (256 x 256 or 128 x 128 blocks for many rows, 32 x 64 for few).  K
// advances 64 at a time, one barrier per step: the next x and W tiles travel into the other half
// of a double-buffered LDS by global_load_lds while the current ones are multiplied.  Within an
// LDS tile row (64 bf16 = 8 chunks of 16 bytes) chunk c of row r sits at position c ^ (r & 7),
// so the 16 rows an operand load touches spread over the banks; the DMA writes LDS linearly, so
// the swizzle is applied by choosing the global chunk each lane fetches.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

constexpr int kLBK = 64;  // k depth of a tile
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
template <int GM, int GN, int WM, int WN>
struct LinTile {
    static constexpr int THREADS = 64 * GM * GN;
    static constexpr int BM = 16 * WM * GM, BN = 16 * WN * GN;
    static constexpr int XT = BM * kLChunks / THREADS;  // x transfers per thread and k tile
    static constexpr int WT = BN * kLChunks / THREADS;  // W transfers per thread and k tile
    static constexpr size_t lds = 2 * (size_t)(BM + BN) * kLBK * 2;  // two buffers of x and W tiles
    static_assert(XT >= 1 && WT >= 1 && XT + WT < 64, "tile transfer counts");
    static_assert(BM * kLChunks % THREADS == 0 && BN * kLChunks % THREADS == 0, "even transfers");
};

template <int GM, int GN, int WM, int WN>
__global__ __launch_bounds__(64 * GM * GN) void linear_kernel(LinearArgs a)
{
    using TL = LinTile<GM, GN, WM, WN>;
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
        for (int i = 0; i < TL::XT; ++i) lds_dma16(xsrc[i] + kt * kLBK, base + (tid + kLThreads * i) * 16);
#pragma unroll
        for (int i = 0; i < TL::WT; ++i) lds_dma16(wsrc[i] + kt * kLBK, base + XB + (tid + kLThreads * i) * 16);
    };

    f4 acc[WM][WN];
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
        for (int j = 0; j < WN; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};

    const int nk = K / kLBK;
    issue(0, 0);
#pragma unroll 1
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this thread's transfers of tile kt have landed
        // Every wave's transfers of tile kt have landed, and every wave is done with tile kt - 1,
        // so the other buffer takes tile kt + 1: one barrier per k tile.
        lds_barrier();
        if (kt + 1 < nk) issue(kt + 1, buf ^ 1);
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

// At most 16 rows (one slot's drafted tokens) and a narrow product: the product is a stream of the
// weight, read once, and the 32 x 64 tiles leave most CUs idle (N = 5120: 80 workgroups).  Here a
// workgroup takes 16 output columns (N / 16 workgroups), its four waves a quarter of the 32-deep k
// steps each, and each wave keeps the fragments of kPF steps in flight while it multiplies the
// previous ones.  No LDS staging: a lane loads its own 16-byte x and W fragments.  The waves'
// partial 16 x 16 tiles are summed in wave order through LDS, and the sums go through the same
// epilogue as the tiled kernel.
constexpr int kSkinnyWaves = 4;
constexpr int kPF = 4;  // k steps of fragments in flight per wave

template <int MT>  // 16-row tiles of x (M <= 16 MT; launched with MT = 1)
__global__ __launch_bounds__(64 * kSkinnyWaves) void linear_skinny_kernel(LinearArgs a)
{
    __shared__ f4 part[kSkinnyWaves - 1][MT][64];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int li = lane & 15, lg = lane >> 4;
    const int K = a.K;
    // columns n0 .. n0 + 15; workgroups are dealt to the 8 XCDs in turn, each XCD taking a
    // contiguous column range (x, read by every workgroup, then sits once in each XCD's L2)
    const int ntiles = gridDim.x, xcd = blockIdx.x % 8, q8 = ntiles / 8, r8 = ntiles % 8;
    const int n0 = 16 * (xcd * q8 + min(xcd, r8) + (int)blockIdx.x / 8);
    // this lane's fragment sources: x row m (rows past M re-read the last one), W row n0 + li
    // (past N the last one); chunk lg of every 32-deep step
    const bf16x8_t *xs[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i)
        xs[i] = reinterpret_cast<const bf16x8_t *>(a.x + (size_t)min(16 * i + li, a.M - 1) * K + 8 * lg);
    const bf16x8_t *ws = reinterpret_cast<const bf16x8_t *>(a.w + (size_t)min(n0 + li, a.N - 1) * K + 8 * lg);
    const int steps = K / 32;
    const int s0 = wave * steps / kSkinnyWaves, mine = (wave + 1) * steps / kSkinnyWaves - s0;
    const int groups = (mine + kPF - 1) / kPF;
    f4 acc[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) acc[i] = f4{0.f, 0.f, 0.f, 0.f};
    // step j of this wave is global step wave + 4 j: 16-byte element offset 4 (wave + 4 j); steps
    // past the wave's count (a wave may have none) load the last step of the row, which is valid,
    // and are not multiplied
    auto at = [&](int j) { return 4 * min(s0 + j, steps - 1); };
    bf16x8_t xa[kPF][MT], wa[kPF];
#pragma unroll
    for (int u = 0; u < kPF; ++u) {
        wa[u] = ws[at(u)];
#pragma unroll
        for (int i = 0; i < MT; ++i) xa[u][i] = xs[i][at(u)];
    }
#pragma unroll 1
    for (int g = 0; g < groups; ++g) {
        bf16x8_t xn[kPF][MT], wn[kPF];
        const int j1 = (g + 1) * kPF;
#pragma unroll
        for (int u = 0; u < kPF; ++u) {  // the next group travels while this one is multiplied
            wn[u] = ws[at(j1 + u)];
#pragma unroll
            for (int i = 0; i < MT; ++i) xn[u][i] = xs[i][at(j1 + u)];
        }
#pragma unroll
        for (int u = 0; u < kPF; ++u)
            if (g * kPF + u < mine)  // uniform over the wave
#pragma unroll
                for (int i = 0; i < MT; ++i) acc[i] = mfma_bf16(xa[u][i], wa[u], acc[i]);
#pragma unroll
        for (int u = 0; u < kPF; ++u) {
            wa[u] = wn[u];
#pragma unroll
            for (int i = 0; i < MT; ++i) xa[u][i] = xn[u][i];
        }
    }
    // the waves' partial tiles, summed in wave order by wave 0
    if (wave > 0)
#pragma unroll
        for (int i = 0; i < MT; ++i) part[wave - 1][i][lane] = acc[i];
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int w = 0; w < kSkinnyWaves - 1; ++w)
#pragma unroll
        for (int i = 0; i < MT; ++i) acc[i] += part[w][i][lane];
    // ---- epilogue: element (row 4 lg + r, column li) of each 16 x 16 tile to its segment
    const int n = n0 + li;
    if (n >= a.N) return;
    int sgi = 0;
#pragma unroll
    for (int q = 1; q < kMaxLinearSegs; ++q)
        if (q < a.n_segs && n >= a.seg[q].n0) sgi = q;
    const LinearSeg &sg = a.seg[sgi];
    const int nc = n - sg.n0;
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = 16 * i + 4 * lg + r;
            if (m >= a.M) continue;
            float v = acc[i][r];
            if (sg.sigmoid) v = 1.0f / (1.0f + expf(-v));
            const size_t o = (size_t)m * sg.ld + nc;
            if (sg.bf16)
                static_cast<uint16_t *>(sg.ptr)[o] = f32_to_bf16(v);
            else
                static_cast<float *>(sg.ptr)[o] = v;
        }
}

template <int MT>
static hipError_t launch_skinny(const LinearArgs &a, hipStream_t stream)
{
    hipLaunchKernelGGL((linear_skinny_kernel<MT>), dim3((unsigned)((a.N + 15) / 16)), dim3(64 * kSkinnyWaves), 0,
                       stream, a);
    return hipGetLastError();
}

template <int GM, int GN, int WM, int WN>
static hipError_t launch_tile(const LinearArgs &a, hipStream_t stream)
{
    using TL = LinTile<GM, GN, WM, WN>;
    const unsigned tiles = (unsigned)((a.N + TL::BN - 1) / TL::BN) * (unsigned)((a.M + TL::BM - 1) / TL::BM);
    const dim3 grid(tiles);
    hipLaunchKernelGGL((linear_kernel<GM, GN, WM, WN>), grid, dim3(TL::THREADS), TL::lds, stream, a);
    return hipGetLastError();
}

// Tile choice.  A k tile brings (BM + BN) x 64 operands into LDS for 2 BM BN x 64 flops, so larger
// workgroup tiles need fewer bytes per flop from L2; 256 x 256 (16 waves of 64 x 64, one workgroup
// per CU) is the fastest per CU, and is taken when its tiles fill at least three quarters of the
// 256 CUs (1024 x 5120 -> 12352: 196 tiles, 134 us against 162 us with 128 x 128).  Otherwise
// 128 x 128 tiles of 16 waves of 32 x 32, two workgroups per CU, spread a smaller product over
// every CU (1024 x 4096 -> 5120: 320 tiles, 56 us against 106 us with 80 of 256 x 256); a few rows
// (one slot's drafted tokens) take 32 x 64 tiles, so the weight stream is spread over enough
// workgroups.
hipError_t launch_linear(const LinearArgs &a, hipStream_t stream)
{
    // At most 16 rows: 16-column workgroups when the 32 x 64 tiles would not give each CU of
    // three quarters of the chip one (16 x 4096 -> 5120: 19 us against 31 us; 16 x 5120 -> 12352,
    // 193 tiles: the tiles, 40 us against 42 us).
    if (a.M <= 16 && (a.N + 63) / 64 < 192) return launch_skinny<1>(a, stream);
    if (a.M <= 64) return launch_tile<2, 2, 1, 2>(a, stream);
    const long big = (long)((a.M + 255) / 256) * ((a.N + 255) / 256);
    if (big >= 192) return launch_tile<4, 4, 4, 4>(a, stream);
    return launch_tile<4, 4, 2, 2>(a, stream);
}

}  // namespace gdn
