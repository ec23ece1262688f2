// bf16 MFMA GEMMs for gfx950, D[t][n] = sum_k A[t][k] * Bt[n][k], with both
// operands K-contiguous (weights are packed once by mla_pack_weight_t):
//   * kv_b_proj decompression (DeepSeek MLA -- Prefix Cache and Chunked
//     Prefill, section 4.4 step 2): A = c_kv rows of the gathered latent,
//     Bt = packed [W_UK | W_UV], output split per head into k_nope and v.
//     It has its own persistent, DMA-fed kernel (decompress_kernel).
//   * the sliced first output projection and the shared second projection of
//     the Local/Global head partition (RedKnot-MLA, sections 1-3, Equation 4),
//     with protected-row replacement fused into the A-operand load
//     (gemm_nt_kernel).
//
// gemm_nt_kernel tiling: 256 threads (4 wavefronts of 64), a TB x TB output
// tile per workgroup (TB = 128, or 64 when 128-wide tiles would leave most
// compute units idle), K in steps of 64 through double-buffered LDS; each
// wavefront owns a TB/2 x TB/2 sub-tile as blocks of v_mfma_f32_32x32x16_bf16.
// The global loads of a k step are issued kPre steps (8 with 64-wide tiles,
// 4 with 128-wide ones) before the step is computed (a ring of register
// slots), so that a long K loop is not paced by one load latency per step. The MFMA is issued as D^T = Bt_frag x A_frag so
// that each lane ends up holding four consecutive output columns of one row,
// which the epilogue packs into 8-byte LDS writes before 16-byte coalesced
// global stores.
#include <algorithm>
#include <mutex>

#include "mla_internal.h"

namespace {

constexpr int BK = 64;
constexpr int kThreads = 256;
constexpr int kLdsK = BK + 8;            // padded row (elements): 144 B, conflict-free b128 reads
constexpr int kTileMin = 128;            // both tile sizes divide multiples of this

// ---------------------------------------------------------------- problem policies

// A = [O_L | O_G] with O_L rows from the artifact or, for protected rows, from
// the recomputation; Bt = packed [W_aL ; W_aG]; D = z.
struct SlicedProjP {
  const uint16_t* art; const uint16_t* rec; const int32_t* prot; int P;
  const uint16_t* glob; int T, HL, HG;
  const uint16_t* wt; int Kt;       // (HL+HG)*128
  uint16_t* z; int ldz;

  __device__ int rows() const { return T; }
  __device__ int K() const { return Kt; }
  // pointers of row t's two column ranges (k < ksplit: the Local part, else
  // the Global part indexed with the global k); t < T
  __device__ void a_rows(int t, const uint16_t*& pl, const uint16_t*& pg, int& ksplit) const {
    ksplit = HL * kDv;
    // binary search of t among the strictly increasing protected rows
    int lo = 0, hi = P;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (prot[mid] < t) lo = mid + 1; else hi = mid;
    }
    const bool is_prot = lo < P && prot[lo] == t;
    pl = is_prot ? rec + (int64_t)lo * HL * kDv : art + (int64_t)t * HL * kDv;
    pg = glob + (int64_t)t * HG * kDv - ksplit;   // indexed with the global k
  }
  __device__ const uint16_t* b_row(int n) const { return wt + (int64_t)n * Kt; }
  __device__ void store(int t, int n, u32x4 val) const {
    *reinterpret_cast<u32x4*>(z + (int64_t)t * ldz + n) = val;
  }
};

// Plain row-major A [T][K] times packed Bt [N][K] into D [T][N].
struct PlainP {
  const uint16_t* a; int T; int Kt; const uint16_t* wt; uint16_t* d; int ldd;

  __device__ int rows() const { return T; }
  __device__ int K() const { return Kt; }
  __device__ void a_rows(int t, const uint16_t*& pl, const uint16_t*& pg, int& ksplit) const {
    pl = a + (int64_t)t * Kt;
    pg = pl;
    ksplit = Kt;
  }
  __device__ const uint16_t* b_row(int n) const { return wt + (int64_t)n * Kt; }
  __device__ void store(int t, int n, u32x4 val) const {
    *reinterpret_cast<u32x4*>(d + (int64_t)t * ldd + n) = val;
  }
};

// ---------------------------------------------------------------- kernel

template <class P, int TB>
__global__ __launch_bounds__(kThreads) void gemm_nt_kernel(P p, int n_mt, int n_nt) {
  constexpr int kTileElems = TB * kLdsK;   // one operand tile
  constexpr int kLdsC = TB + 8;            // padded epilogue row
  constexpr int RPT = TB / 32;             // rows each thread loads per operand
  constexpr int NBK = TB / 64;             // 32 x 32 blocks per wavefront and dimension
  constexpr int kPre = TB == 64 ? 8 : 4;   // k steps whose loads are in flight
  static_assert(TB * kLdsC <= 4 * kTileElems, "epilogue tile fits the operand buffers");
  __shared__ __attribute__((aligned(16))) uint16_t lds[4 * kTileElems];   // A0 B0 A1 B1
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, g = lane >> 5;

  // tile of this workgroup (m fastest within an XCD's contiguous range)
  const uint32_t work = xcd_remap(blockIdx.x, (uint32_t)(n_mt * n_nt));
  const int mt = (int)(work % (uint32_t)n_mt);
  const int nt = (int)(work / (uint32_t)n_mt);
  const int t0 = mt * TB, n0 = nt * TB;

  // each thread loads RPT rows x one 16-byte vector of the A and B tiles per k step
  const int lrow = tid >> 3, lvec = tid & 7;
  // Rows past the last one load row M-1 and are zeroed when written to LDS,
  // so no load is predicated (the compiler then tracks each slot's loads
  // exactly and waits only for the slot it moves into LDS).
  const int M = p.rows();
  const uint16_t* apl[RPT];
  const uint16_t* apg[RPT];
  const uint16_t* bp[RPT];
  bool aval[RPT];
  int ksplit = 0;
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int t = t0 + lrow + 32 * i;
    aval[i] = t < M;
    p.a_rows(min(t, M - 1), apl[i], apg[i], ksplit);
    bp[i] = p.b_row(n0 + lrow + 32 * i);
  }
  const int K = p.K();
  const int nk = K / BK;

  u32x4 ra[kPre][RPT], rb[kPre][RPT];
  auto gload = [&](int slot, int kt) __attribute__((always_inline)) {
    const int k = kt * BK + lvec * 8;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const uint16_t* src = k < ksplit ? apl[i] : apg[i];
      ra[slot][i] = *reinterpret_cast<const u32x4*>(src + k);
      rb[slot][i] = *reinterpret_cast<const u32x4*>(bp[i] + k);
    }
  };
  auto lstore = [&](int slot, int buf) __attribute__((always_inline)) {
    uint16_t* As = lds + (2 * buf) * kTileElems;
    uint16_t* Bs = lds + (2 * buf + 1) * kTileElems;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      *reinterpret_cast<u32x4*>(As + (lrow + 32 * i) * kLdsK + lvec * 8) =
          aval[i] ? ra[slot][i] : u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(Bs + (lrow + 32 * i) * kLdsK + lvec * 8) = rb[slot][i];
    }
  };

  f32x16 acc[NBK][NBK];
#pragma unroll
  for (int a = 0; a < NBK; ++a)
#pragma unroll
    for (int b = 0; b < NBK; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.f;

  auto compute = [&](int buf) __attribute__((always_inline)) {
    const uint16_t* As = lds + (2 * buf) * kTileElems;
    const uint16_t* Bs = lds + (2 * buf + 1) * kTileElems;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8 af[NBK], bfr[NBK];
#pragma unroll
      for (int tb = 0; tb < NBK; ++tb)
        af[tb] = *reinterpret_cast<const bf16x8*>(As + (wm * (TB / 2) + tb * 32 + l32) * kLdsK + ks * 16 + g * 8);
#pragma unroll
      for (int nb = 0; nb < NBK; ++nb)
        bfr[nb] = *reinterpret_cast<const bf16x8*>(Bs + (wn * (TB / 2) + nb * 32 + l32) * kLdsK + ks * 16 + g * 8);
#pragma unroll
      for (int nb = 0; nb < NBK; ++nb)
#pragma unroll
        for (int tb = 0; tb < NBK; ++tb)
          acc[nb][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[nb], af[tb], acc[nb][tb], 0, 0, 0);
    }
  };

  // Step kt: refill slot kt % kPre with the loads of step kt + kPre, compute
  // step kt from LDS buffer kt & 1, move step kt + 1 from its register slot
  // into the other buffer (last read in step kt - 1, before the previous
  // barrier), then meet the other wavefronts. Steps past the last are
  // clamped to it (loaded again, never computed), so every step issues the
  // same loads.
#pragma unroll
  for (int s2 = 0; s2 < kPre; ++s2) gload(s2, min(s2, nk - 1));
  lstore(0, 0);
  __syncthreads();
  for (int kt0 = 0; kt0 < nk; kt0 += kPre) {
#pragma unroll
    for (int u = 0; u < kPre; ++u) {
      const int kt = kt0 + u;
      if (kt < nk) {
        gload(u, min(kt + kPre, nk - 1));
        compute(u & 1);
        lstore((u + 1) % kPre, (u + 1) & 1);
        __syncthreads();
      }
    }
  }

  // epilogue: lane holds D^T rows n = 8*(i/4) + 4*g + (i%4), column t = l32
  uint16_t* Cs = lds;
#pragma unroll
  for (int nb = 0; nb < NBK; ++nb)
#pragma unroll
    for (int tb = 0; tb < NBK; ++tb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int t = wm * (TB / 2) + tb * 32 + l32;
        const int n = wn * (TB / 2) + nb * 32 + 8 * q + 4 * g;
        u32x2 w;
        w.x = pack_bf16x2(acc[nb][tb][4 * q + 0], acc[nb][tb][4 * q + 1]);
        w.y = pack_bf16x2(acc[nb][tb][4 * q + 2], acc[nb][tb][4 * q + 3]);
        *reinterpret_cast<u32x2*>(Cs + t * kLdsC + n) = w;
      }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < (TB * TB / 8) / kThreads; ++i) {
    const int idx = tid + i * kThreads;
    const int r = idx / (TB / 8), vec = idx % (TB / 8);
    if (t0 + r < M) p.store(t0 + r, n0 + vec * 8, *reinterpret_cast<const u32x4*>(Cs + r * kLdsC + vec * 8));
  }
}

template <class P>
int launch_gemm(const P& p, int M, int N, hipStream_t s, const char* what) {
  // 128-wide tiles unless they would give fewer workgroups than compute units
  const int ncu = std::max(mla_num_cus(), 1);
  const int64_t big = (int64_t)((M + 127) / 128) * (N / 128);
  if (big >= ncu) {
    const int n_mt = (M + 127) / 128, n_nt = N / 128;
    MLA_REQUIRE(big < (int64_t)1 << 31, MLA_ERR_INVALID_ARG, "%s: problem too large", what);
    hipLaunchKernelGGL((gemm_nt_kernel<P, 128>), dim3((unsigned)big), dim3(kThreads), 0, s, p, n_mt, n_nt);
  } else {
    const int n_mt = (M + 63) / 64, n_nt = N / 64;
    hipLaunchKernelGGL((gemm_nt_kernel<P, 64>), dim3((unsigned)(n_mt * n_nt)), dim3(kThreads), 0, s, p, n_mt, n_nt);
  }
  return mla_check_launch(what);
}

// ---------------------------------------------------------------- decompression kernel
//
// Persistent: one workgroup of 8 wavefronts per CU walks 256 x 256 output
// tiles (tokens x columns). Each wavefront owns a 64 x 128 sub-tile, held as
// 2 x 4 blocks of v_mfma_f32_32x32x16_bf16 accumulators and issued as D^T =
// W_frag x A_frag, so a lane holds four consecutive output columns of one
// token. A wavefront's 128 columns are always one head's W_UK or W_UV, also
// when a tile straddles the W_UK / W_UV boundary.
//
// Operands go from HBM straight into LDS (global_load_lds, no register
// staging) in k steps of 64 through two LDS stages of 64 KB; each DMA
// instruction moves 8 rows x 128 B, whole cache lines (k steps of 32, which
// give 64-byte row pieces, measured 6% slower with twice the L2 requests).
// The pipeline runs over the flattened (tile, k step) sequence of the
// workgroup, so the first step of the next tile is already in flight while a
// tile finishes. LDS rows carry no padding: chunks are XOR-swizzled within a
// row (dec_swz) so that every 16-lane group of a fragment read hits 16
// distinct 16-byte bank groups.
//
// Epilogue: one v_permlane32_swap per register pair gives each lane eight
// consecutive bf16 columns of one token; a 4 KB LDS slice per wavefront (the
// 32 KB beside the two stages) regroups 16 tokens at a time so that each
// 16-byte buffer store instruction writes four whole 256-byte rows (rows past
// the last token are dropped by the buffer range check). Stores that wrote
// 32 bytes into each of 32 rows measured 3-8% slower. The stores are
// non-temporal, which measured 2.5-6.5% faster than the default policy with
// whole-row stores (and 3% slower with the scattered ones). The stores of a tile
// are issued in the first step of the next tile, after that step's DMA, so
// they overlap its products.
//
// Completion of the DMA is tracked with the vector-memory counter, which
// counts the buffer stores too. Vector memory operations report completion to
// the wavefront in issue order, so a step waits until no more operations are
// outstanding than were issued after its own DMA: the DMAs of the steps
// already prefetched beyond it, plus the 16 stores of the previous tile when
// those were issued after this step's DMA (the first kDNS-1 steps after a
// tile boundary). Every wavefront issues exactly kDDma DMAs per step and 16
// stores per tile, with no predication, so the count is exact.
constexpr int kDT = 256;                       // tile edge (tokens and columns)
constexpr int kDBK = 64;                       // k step
constexpr int kDSteps = kDc / kDBK;            // k steps per tile
constexpr int kDNS = 2;                        // LDS stages
constexpr int kDRow = kDBK * 2;                // bytes per row in LDS
constexpr int kDChunks = kDRow / 16;           // 16-byte chunks per row
constexpr int kDRowsPerDma = 64 / kDChunks;    // rows covered by one DMA instruction
constexpr int kDOpB = kDT * kDRow;             // bytes per operand per stage
constexpr int kDStageB = 2 * kDOpB;            // bytes per stage (A then W)
constexpr int kDThreads = 512;
constexpr int kDDmaOp = kDOpB / 1024 / 8;      // DMA instructions per wavefront per operand per step
constexpr int kDDma = 2 * kDDmaOp;             // DMA instructions per wavefront per step
constexpr int kDStores = 16;                   // stores per wavefront per tile
constexpr int kDEpB = 16 * 256;                // epilogue LDS bytes per wavefront (16 tokens x 128 columns)
static_assert(kDNS * kDStageB + 8 * kDEpB <= 160 * 1024 && (kDNS & (kDNS - 1)) == 0 && (kDSteps & (kDSteps - 1)) == 0,
              "decompression LDS ring");

// fp8 (e4m3) A operand: rows of 64 bytes (one k step of codes), 4 chunks
constexpr int kDRow8 = kDBK;                   // bytes per A row in LDS (fp8)
constexpr int kDChunks8 = kDRow8 / 16;
constexpr int kDRowsPerDma8 = 64 / kDChunks8;
constexpr int kDOpB8 = kDT * kDRow8;           // A bytes per stage (fp8)
constexpr int kDDmaOp8 = kDOpB8 / 1024 / 8;

// LDS position of chunk c of row r: rows are swizzled so that the 16 rows
// read by 16 consecutive lanes (same chunk) fall on 16 distinct 16-byte bank
// groups of a 256-byte bank line
__device__ __forceinline__ int dec_swz(int r, int c) {
  return c ^ ((r / (16 / kDChunks)) % kDChunks);
}
// the same for 64-byte fp8 rows: four rows share a bank line, and rows
// 4 apart put a chunk on different bank groups
__device__ __forceinline__ int dec_swz8(int r, int c) { return c ^ ((r >> 2) & 3); }

// 8 e4m3 codes (two dwords) -> 8 bf16, exactly (v_cvt_scalef32_pk_bf16_fp8
// with scale 1: every e4m3 value, subnormals included, is a bf16 value)
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(u32x2 c) {
  typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
  const bf16x2v p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)c.x, 1.0f, false);
  const bf16x2v p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)c.x, 1.0f, true);
  const bf16x2v p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)c.y, 1.0f, false);
  const bf16x2v p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)c.y, 1.0f, true);
  return bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

struct DecArgs {
  const uint16_t* lat; int64_t ld; int M;
  const float* scale;                           // fp8 A: per-token scale, else unused
  const uint16_t* wt; int H_total, h_begin, Hsel;
  uint16_t* k; int64_t khs; uint16_t* v; int64_t vhs;
  int n_mt, n_nt;
};

// rank (0 .. n_mt*n_nt-1) -> (token tile, column tile): consecutive ranks
// walk kGroupM token tiles x all column tiles, so the 32 workgroups of one
// XCD, which take consecutive ranks together, share 6 latent tiles and 5-6
// weight tiles (3 MB) in that XCD's L2. Groups of 3 to 10 token tiles
// measured alike; powers of two (2, 4, 8) were 10-13% slower on some shapes
// (16384 tokens x 128 heads, and 8 heads).
__device__ __forceinline__ void dec_tile(int rank, int n_mt, int n_nt, int& mt, int& nt) {
  constexpr int kGroupM = 6;
  const int per_group = kGroupM * n_nt;
  const int first_mt = (rank / per_group) * kGroupM;
  const int gm = min(n_mt - first_mt, kGroupM);
  const int in_group = rank % per_group;
  mt = first_mt + in_group % gm;
  nt = in_group / gm;
}

// kFp8A: the A rows are e4m3 codes (their first 512 bytes), DMA'd to LDS as
// bytes and widened to bf16 at the fragment read (exactly); the token's
// scale multiplies the fp32 sums in the epilogue.
template <bool kFp8A>
__global__ __launch_bounds__(kDThreads, 1) void decompress_kernel(DecArgs a) {
  constexpr int kARow = kFp8A ? kDRow8 : kDRow;           // A bytes per LDS row
  constexpr int kAOp = kFp8A ? kDOpB8 : kDOpB;            // A bytes per stage
  constexpr int kAChunks = kFp8A ? kDChunks8 : kDChunks;
  constexpr int kARowsPerDma = kFp8A ? kDRowsPerDma8 : kDRowsPerDma;
  constexpr int kADma = kFp8A ? kDDmaOp8 : kDDmaOp;       // A DMA instructions per wavefront per step
  constexpr int kStageB = kAOp + kDOpB;                   // bytes per stage (A then W)
  extern __shared__ __attribute__((aligned(1024))) uint8_t dlds[];   // kDNS stages
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;      // 4 x 2 wavefronts: 64 tokens x 128 columns each
  const int l32 = lane & 31, g = lane >> 5;
  const int HK = a.Hsel * kDnope;               // columns of the K part

  // This workgroup's ranks: XCD x (= blockIdx % 8) owns a contiguous range of
  // ranks, which its workgroups take round-robin.
  const int total = a.n_mt * a.n_nt;
  const int G = gridDim.x;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int nslots = (G - xcd + 7) >> 3;        // workgroups on this XCD
  const int chunk = (total + 7) >> 3;
  const int rbeg = min(xcd * chunk, total), rend = min(rbeg + chunk, total);
  const int my_tiles = rbeg + slot < rend ? (rend - rbeg - slot + nslots - 1) / nslots : 0;
  const int nsteps = my_tiles * kDSteps;
  if (nsteps == 0) return;

  // DMA source of this lane for the tile being prefetched: per-lane 32-bit
  // byte offsets (row kDRowsPerDma * i + lane / kDChunks of instruction
  // i = 8 i2 + wave, chunk lane % kDChunks at its swizzled position), fixed
  // for the tile; the k step only moves the uniform base.
  uint32_t aof[kADma], bof[kDDmaOp];
  auto set_dma_tile = [&](int j) __attribute__((always_inline)) {
    int mt, nt;
    dec_tile(rbeg + slot + j * nslots, a.n_mt, a.n_nt, mt, nt);
#pragma unroll
    for (int i2 = 0; i2 < kADma; ++i2) {
      const int r = kARowsPerDma * (i2 * 8 + wave) + lane / kAChunks;
      const int gc = kFp8A ? dec_swz8(r, lane % kAChunks) : dec_swz(r, lane % kAChunks);
      const int t = min(mt * kDT + r, a.M - 1);
      aof[i2] = (uint32_t)t * (uint32_t)(a.ld * 2) + gc * 16;
    }
#pragma unroll
    for (int i2 = 0; i2 < kDDmaOp; ++i2) {
      const int r = kDRowsPerDma * (i2 * 8 + wave) + lane / kDChunks;
      const int gc = dec_swz(r, lane % kDChunks);
      const int n = nt * kDT + r;               // output column -> packed weight row
      const int wrow = n < HK ? a.h_begin * kDnope + n : a.H_total * kDnope + a.h_begin * kDnope + (n - HK);
      bof[i2] = (uint32_t)wrow * (kDc * 2) + gc * 16;
    }
  };
  // (tile, k step) of the next DMA; past the last step it stays there, so the
  // clamped copies re-read valid data
  int dj = 0, dkk = 0;
  set_dma_tile(0);
  auto dma_next = [&](int stage) __attribute__((always_inline)) {
    uint8_t* st = dlds + stage * kStageB;
    const uint8_t* sa = reinterpret_cast<const uint8_t*>(a.lat) + dkk * kARow;
    const uint8_t* sb = reinterpret_cast<const uint8_t*>(a.wt) + dkk * (kDBK * 2);
#pragma unroll
    for (int i2 = 0; i2 < kADma; ++i2) dma16s(sa, aof[i2], st + (i2 * 8 + wave) * 1024);
#pragma unroll
    for (int i2 = 0; i2 < kDDmaOp; ++i2) dma16s(sb, bof[i2], st + kAOp + (i2 * 8 + wave) * 1024);
    if (++dkk == kDSteps) {
      if (dj + 1 < my_tiles) {
        dkk = 0;
        set_dma_tile(++dj);
      } else {
        dkk = kDSteps - 1;
      }
    }
  };

  // fragment read offsets (bytes in a stage) for the 16-wide k sub-steps
  constexpr int kSub = kDBK / 16;
  int aoff[kSub], boff[kSub];
#pragma unroll
  for (int s2 = 0; s2 < kSub; ++s2) {
    // bf16 rows: sub-step s2 takes k = 16 s2 + 8 g .. + 7 in lane half g.
    // fp8 rows: lane half g reads all 16 codes of chunk (s2 & ~1) + g with
    // one 16-byte read (8-byte reads of half a chunk use half the banks and
    // conflict two ways); codes 0-7 feed sub-step s2 & ~1, codes 8-15 the
    // next one, so sub-step s2 takes k = 16 ((s2 & ~1) + g) + 8 (s2 & 1) ..
    // + 7, and the weight fragments are read for the same k.
    const int bchunk = kFp8A ? 2 * ((s2 & ~1) + g) + (s2 & 1) : 2 * s2 + g;
    aoff[s2] = kFp8A ? (wm * 64 + l32) * kDRow8 + dec_swz8(l32, (s2 & ~1) + g) * 16
                     : (wm * 64 + l32) * kDRow + dec_swz(l32, 2 * s2 + g) * 16;
    boff[s2] = kAOp + (wn * 128 + l32) * kDRow + dec_swz(l32, bchunk) * 16;
  }

  f32x16 acc[4][2];
  // fp8 A: the scales of this lane's two tokens of the tile being computed,
  // loaded in the tile's first step (after that step's DMA and the previous
  // tile's stores, so the step waits that follow count them in order) and
  // used by its epilogue
  float tile_scale[2] = {1.f, 1.f};
  auto load_scales = [&](int j) __attribute__((always_inline)) {
    int mt, nt;
    dec_tile(rbeg + slot + j * nslots, a.n_mt, a.n_nt, mt, nt);
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) tile_scale[tb] = a.scale[min(mt * kDT + wm * 64 + tb * 32 + l32, a.M - 1)];
  };
  auto zero = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[nb][tb][i] = 0.f;
  };

  // Epilogue of the tile with flattened index j: 16 buffer stores per lane,
  // each writing four whole 256-byte rows (this wavefront's 128 columns of
  // four tokens). The accumulators are regrouped through a 4 KB LDS slice per
  // wavefront, 16 tokens at a time.
  uint8_t* ep = dlds + kDNS * kStageB + wave * kDEpB;
  auto store_tile = [&](int j) __attribute__((always_inline)) {
    int mt, nt;
    dec_tile(rbeg + slot + j * nslots, a.n_mt, a.n_nt, mt, nt);
    if constexpr (kFp8A) {
      // the fp32 sums of this lane's token (column l32 of token block tb)
      // times the token's scale, before the bf16 rounding
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[nb][tb][i] *= tile_scale[tb];
    }
    const int n0 = nt * kDT + wn * 128;         // first column of this wavefront
    const bool is_v = n0 >= HK;
    const int hs = (is_v ? n0 - HK : n0) / kDnope;
    uint16_t* dst = is_v ? a.v + (int64_t)hs * a.vhs : a.k + (int64_t)hs * a.khs;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(dst, (short)0, a.M * (kDnope * 2), 0x00020000);
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      u32x4 val[8];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          // lane g holds columns 8q + 4g .. +3 of q = 2p, 2p+1; after the swap
          // lane g = 0 holds all 8 columns of q = 2p+1, lane g = 1 those of q = 2p
          uint32_t x0 = cvt_pk_bf16(acc[nb][tb][8 * p + 0], acc[nb][tb][8 * p + 1]);
          uint32_t y0 = cvt_pk_bf16(acc[nb][tb][8 * p + 2], acc[nb][tb][8 * p + 3]);
          uint32_t x1 = cvt_pk_bf16(acc[nb][tb][8 * p + 4], acc[nb][tb][8 * p + 5]);
          uint32_t y1 = cvt_pk_bf16(acc[nb][tb][8 * p + 6], acc[nb][tb][8 * p + 7]);
          const auto sx = __builtin_amdgcn_permlane32_swap(x1, x0, false, false);
          const auto sy = __builtin_amdgcn_permlane32_swap(y1, y0, false, false);
          val[nb * 2 + p] = u32x4{sx[0], sy[0], sx[1], sy[1]};
        }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        // tokens 16h .. 16h+15 of this block: their lanes write 16-byte chunk
        // c of row r at position c ^ r (conflict-free writes and reads)
        if ((l32 >> 4) == h) {
          const int r = l32 & 15;
#pragma unroll
          for (int nb = 0; nb < 4; ++nb)
#pragma unroll
            for (int p = 0; p < 2; ++p) {
              const int c = nb * 4 + 2 * p + 1 - g;
              *reinterpret_cast<u32x4*>(ep + r * 256 + ((c ^ r) << 4)) = val[nb * 2 + p];
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = i * 4 + (lane >> 4), c = lane & 15;
          const u32x4 x = *reinterpret_cast<const u32x4*>(ep + r * 256 + ((c ^ r) << 4));
          const int t = mt * kDT + wm * 64 + tb * 32 + h * 16 + r;
          // non-temporal (cache policy bit 1): the 1 GB output stream is not kept in L2
          __builtin_amdgcn_raw_buffer_store_b128(x, rs, t * (kDnope * 2) + c * 16, 0, 2);
        }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
      }
    }
  };

  // Pipeline: step s waits for its own DMA, meets the other wavefronts at the
  // barrier (then stage s % kDNS is complete and stage (s-1) % kDNS is no
  // longer read), issues the DMA of step s+kDNS-1 into that stage and
  // computes step s.
  // Steps past the end are clamped to the last step: the copy goes into a
  // stage no later step reads, and every step issues the same number of DMAs.
#pragma unroll
  for (int s = 0; s < kDNS - 1; ++s) dma_next(s);
  zero();
#pragma unroll 1
  for (int s = 0; s < nsteps; ++s) {
    const int kk = s & (kDSteps - 1);
    if (s >= kDSteps && kk >= 1 && kk <= kDNS - 1) wait_vmcnt<(kDNS - 2) * kDDma + kDStores>();
    else wait_vmcnt<(kDNS - 2) * kDDma>();
    __syncthreads();
    dma_next((s + kDNS - 1) & (kDNS - 1));
    if (kk == 0 && s > 0) {
      store_tile(s / kDSteps - 1);
      zero();
    }
    if constexpr (kFp8A)
      if (kk == 0) load_scales(s / kDSteps);
    const uint8_t* st = dlds + (s & (kDNS - 1)) * kStageB;
    u32x4 a16[2];                              // fp8: the 16 codes of two sub-steps
#pragma unroll
    for (int s2 = 0; s2 < kSub; ++s2) {
      bf16x8 af[2], bf[4];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        if constexpr (kFp8A) {
          if ((s2 & 1) == 0) a16[tb] = *reinterpret_cast<const u32x4*>(st + aoff[s2] + tb * 32 * kDRow8);
          af[tb] = e4m3x8_to_bf16((s2 & 1) ? u32x2{a16[tb].z, a16[tb].w} : u32x2{a16[tb].x, a16[tb].y});
        } else {
          af[tb] = *reinterpret_cast<const bf16x8*>(st + aoff[s2] + tb * 32 * kDRow);
        }
      }
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) bf[nb] = *reinterpret_cast<const bf16x8*>(st + boff[s2] + nb * 32 * kDRow);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
          acc[nb][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[nb], af[tb], acc[nb][tb], 0, 0, 0);
    }
  }
  store_tile(my_tiles - 1);
  // no DMA may still be writing LDS when the workgroup ends
  wait_vmcnt<0>();
}

// ---------------------------------------------------------------- weight pack (transpose)

constexpr int kTr = 64;
__global__ __launch_bounds__(256) void transpose_kernel(const uint16_t* __restrict__ w, int K, int N,
                                                         uint16_t* __restrict__ out) {
  __shared__ uint16_t tile[kTr][kTr + 2];
  const int k0 = blockIdx.y * kTr, n0 = blockIdx.x * kTr;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int r = ty; r < kTr; r += 4) {
    const int k = k0 + r, n = n0 + tx;
    tile[r][tx] = (k < K && n < N) ? w[(int64_t)k * N + n] : 0;
  }
  __syncthreads();
  for (int r = ty; r < kTr; r += 4) {
    const int n = n0 + r, k = k0 + tx;
    if (n < N && k < K) out[(int64_t)n * K + k] = tile[tx][r];
  }
}

}  // namespace

extern "C" int mla_pack_weight_t(const void* w, int K, int N, void* out, void* stream) {
  mla_begin_call();
  MLA_REQUIRE(w && out, MLA_ERR_INVALID_ARG, "mla_pack_weight_t: null pointer argument");
  MLA_REQUIRE(K > 0 && N > 0 && K % 8 == 0 && N % 8 == 0, MLA_ERR_INVALID_ARG,
              "mla_pack_weight_t: K (%d) and N (%d) must be positive multiples of 8", K, N);
  MLA_REQUIRE(w != out, MLA_ERR_INVALID_ARG, "mla_pack_weight_t: in-place transpose is not supported");
  dim3 g((N + kTr - 1) / kTr, (K + kTr - 1) / kTr);
  hipLaunchKernelGGL(transpose_kernel, g, dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                     static_cast<const uint16_t*>(w), K, N, static_cast<uint16_t*>(out));
  return mla_check_launch("mla_pack_weight_t");
}

extern "C" int mla_decompress(const void* latent, int64_t ld_latent, const float* row_scale, int n_tokens,
                              const void* w_t, int H_total, int h_begin, int h_end,
                              void* k_nope, int64_t k_head_stride,
                              void* v, int64_t v_head_stride, void* stream) {
  mla_begin_call();
  MLA_REQUIRE(n_tokens >= 0, MLA_ERR_INVALID_ARG, "mla_decompress: n_tokens must be >= 0");
  MLA_REQUIRE(H_total > 0 && 0 <= h_begin && h_begin < h_end && h_end <= H_total, MLA_ERR_INVALID_ARG,
              "mla_decompress: need 0 <= h_begin (%d) < h_end (%d) <= H_total (%d)", h_begin, h_end, H_total);
  if (n_tokens == 0) return MLA_OK;
  MLA_REQUIRE(latent && w_t && k_nope && v, MLA_ERR_INVALID_ARG, "mla_decompress: null pointer argument");
  MLA_REQUIRE(!row_scale || (reinterpret_cast<uintptr_t>(row_scale) & 3u) == 0, MLA_ERR_INVALID_ARG,
              "mla_decompress: row_scale must be 4-byte aligned");
  MLA_REQUIRE(mla_aligned16(latent) && mla_aligned16(w_t) && mla_aligned16(k_nope) && mla_aligned16(v),
              MLA_ERR_INVALID_ARG, "mla_decompress: pointers must be 16-byte aligned");
  MLA_REQUIRE(ld_latent >= kDc && ld_latent % 8 == 0, MLA_ERR_INVALID_ARG,
              "mla_decompress: ld_latent (%lld) must be >= 512 and a multiple of 8", (long long)ld_latent);
  // the kernel addresses the latent and the packed weight with 32-bit byte
  // offsets and each head's output with a 31-bit buffer range
  MLA_REQUIRE((int64_t)n_tokens * ld_latent * 2 < ((int64_t)1 << 32) && (int64_t)n_tokens * kDnope * 2 < ((int64_t)1 << 31),
              MLA_ERR_UNSUPPORTED, "mla_decompress: n_tokens (%d) too large for one call; split the tokens", n_tokens);
  MLA_REQUIRE((int64_t)H_total * 2 * kDnope * kDc * 2 < ((int64_t)1 << 32), MLA_ERR_UNSUPPORTED,
              "mla_decompress: H_total (%d) too large", H_total);
  const int Hsel = h_end - h_begin;
  MLA_REQUIRE(k_head_stride >= (int64_t)n_tokens * kDnope && v_head_stride >= (int64_t)n_tokens * kDv &&
                  k_head_stride % 8 == 0 && v_head_stride % 8 == 0,
              MLA_ERR_INVALID_ARG, "mla_decompress: head strides must be >= n_tokens*128 and multiples of 8");
  DecArgs d{static_cast<const uint16_t*>(latent), ld_latent, n_tokens, row_scale,
            static_cast<const uint16_t*>(w_t), H_total, h_begin, Hsel,
            static_cast<uint16_t*>(k_nope), k_head_stride, static_cast<uint16_t*>(v), v_head_stride,
            (n_tokens + kDT - 1) / kDT, Hsel * 2 * kDnope / kDT};
  const int64_t total = (int64_t)d.n_mt * d.n_nt;
  MLA_REQUIRE(total < (int64_t)1 << 31, MLA_ERR_INVALID_ARG, "mla_decompress: problem too large");
  const bool fp8 = row_scale != nullptr;
  const size_t lds = (size_t)kDNS * (fp8 ? kDOpB8 + kDOpB : kDStageB) + 8 * kDEpB;
  const void* kern = fp8 ? reinterpret_cast<const void*>(&decompress_kernel<true>)
                         : reinterpret_cast<const void*>(&decompress_kernel<false>);
  if (hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess) {
    mla_set_error("mla_decompress: cannot reserve %zu bytes of LDS", lds);
    return MLA_ERR_LAUNCH;
  }
  // persistent grid: one workgroup per compute unit, none without a tile
  const int ncu = mla_num_cus();
  MLA_REQUIRE(ncu > 0, MLA_ERR_LAUNCH, "mla_decompress: cannot query the compute-unit count");
  const unsigned grid = (unsigned)std::min<int64_t>(total, ncu);
  if (fp8)
    hipLaunchKernelGGL(decompress_kernel<true>, dim3(grid), dim3(kDThreads), lds,
                       reinterpret_cast<hipStream_t>(stream), d);
  else
    hipLaunchKernelGGL(decompress_kernel<false>, dim3(grid), dim3(kDThreads), lds,
                       reinterpret_cast<hipStream_t>(stream), d);
  return mla_check_launch("mla_decompress");
}

namespace {

// Sliced projection then shared projection through the intermediate z
// (bf16 [T][d_mid], device memory of at least T * d_mid elements).
int head_partition_merge_impl(const void* art_out, const void* rec_out, const int32_t* prot_rows, int P,
                              const void* glob_out, const void* wa_t, const void* wb_t, int T, int HL, int HG,
                              int d_mid, int d_model, void* z, void* y, void* stream, const char* name) {
  MLA_REQUIRE(T >= 0 && P >= 0 && P <= T && HL >= 0 && HG >= 0 && HL + HG > 0, MLA_ERR_INVALID_ARG,
              "%s: need T >= 0, 0 <= P <= T, HL, HG >= 0, HL + HG > 0", name);
  if (T == 0) return MLA_OK;
  MLA_REQUIRE(wa_t && wb_t && z && y && (HL == 0 || art_out) && (HG == 0 || glob_out) &&
                  (P == 0 || (rec_out && prot_rows)),
              MLA_ERR_INVALID_ARG, "%s: null pointer argument", name);
  MLA_REQUIRE(d_mid > 0 && d_model > 0 && d_mid % kTileMin == 0 && d_model % kTileMin == 0, MLA_ERR_UNSUPPORTED,
              "%s: d_mid (%d) and d_model (%d) must be multiples of 128", name, d_mid, d_model);
  MLA_REQUIRE((HL * kDv) % BK == 0, MLA_ERR_UNSUPPORTED, "%s: HL*128 must be a multiple of 64", name);
  const void* ptrs[] = {art_out, rec_out, glob_out, wa_t, wb_t, z, y};
  for (const void* q : ptrs) MLA_REQUIRE(!q || mla_aligned16(q), MLA_ERR_INVALID_ARG,
                                         "%s: pointers must be 16-byte aligned", name);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  SlicedProjP p1{static_cast<const uint16_t*>(art_out), static_cast<const uint16_t*>(rec_out), prot_rows, P,
                 static_cast<const uint16_t*>(glob_out), T, HL, HG, static_cast<const uint16_t*>(wa_t),
                 (HL + HG) * kDv, static_cast<uint16_t*>(z), d_mid};
  int rc = launch_gemm(p1, T, d_mid, s, name);
  if (rc != MLA_OK) return rc;
  PlainP p2{static_cast<const uint16_t*>(z), T, d_mid, static_cast<const uint16_t*>(wb_t),
            static_cast<uint16_t*>(y), d_model};
  return launch_gemm(p2, T, d_model, s, name);
}

}  // namespace

extern "C" int mla_head_partition_merge(const void* art_out, const void* rec_out,
                                        const int32_t* prot_rows, int P, const void* glob_out,
                                        const void* wa_t, const void* wb_t, int T, int HL, int HG,
                                        int d_mid, int d_model, void* z, void* y, void* stream) {
  mla_begin_call();
  return head_partition_merge_impl(art_out, rec_out, prot_rows, P, glob_out, wa_t, wb_t, T, HL, HG, d_mid,
                                   d_model, z, y, stream, "mla_head_partition_merge");
}

// ---------------------------------------------------------------- no-allocation variant
//
// The intermediate z of mla_head_partition_merge_noalloc lives in this
// file-scope device array: one copy per device, loaded with the code object
// and held until the process ends. Host code never passes its name to a
// kernel (on the host the name is only a stand-in); it takes the device
// address of the current device's copy with hipGetSymbolAddress, once per
// device, and uses that address.
constexpr int64_t kHpmScratchBytes = (int64_t)8 << 20;
static __device__ __align__(256) uint8_t scratch[kHpmScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};

// device address of the current device's scratch array, or nullptr (with
// the error message set)
void* scratch_on_current_device(const char* name) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    mla_set_error("%s: cannot tell the current device", name);
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_addr[dev] == nullptr) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) {
      mla_set_error("%s: hipGetSymbolAddress of the scratch array failed on device %d: %s", name, dev,
                    hipGetErrorString(e));
      return nullptr;
    }
    g_scratch_addr[dev] = ptr;
  }
  return g_scratch_addr[dev];
}

}  // namespace

extern "C" int mla_head_partition_merge_noalloc(const void* art_out, const void* rec_out,
                                                const int32_t* prot_rows, int P, const void* glob_out,
                                                const void* wa_t, const void* wb_t, int T, int HL, int HG,
                                                int d_mid, int d_model, void* y, void* stream) {
  mla_begin_call();
  const char* name = "mla_head_partition_merge_noalloc";
  MLA_REQUIRE(T >= 0 && d_mid > 0, MLA_ERR_INVALID_ARG, "%s: need T >= 0 and d_mid > 0", name);
  MLA_REQUIRE((int64_t)T * d_mid * 2 <= kHpmScratchBytes, MLA_ERR_INVALID_ARG,
              "%s: T * d_mid (%lld) exceeds the scratch array's %lld bf16 elements; use "
              "mla_head_partition_merge with a workspace",
              name, (long long)T * d_mid, (long long)(kHpmScratchBytes / 2));
  if (T == 0) return head_partition_merge_impl(art_out, rec_out, prot_rows, P, glob_out, wa_t, wb_t, T, HL, HG,
                                               d_mid, d_model, nullptr, y, stream, name);
  void* z = scratch_on_current_device(name);
  if (!z) return MLA_ERR_LAUNCH;
  return head_partition_merge_impl(art_out, rec_out, prot_rows, P, glob_out, wa_t, wb_t, T, HL, HG, d_mid,
                                   d_model, z, y, stream, name);
}
