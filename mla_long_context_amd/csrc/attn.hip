// Flash-attention prefill returning (out, lse) for MLA on gfx950: the context
// pass (no mask) and the causal extend pass of the two-stage prefill
// (DeepSeek MLA -- Prefix Cache and Chunked Prefill, sections 4.2 and 4.4
// steps 3-4). Keys are K = [k_nope (per head, 128) | k_rope (64, one per token,
// shared by every head)]; values are per head, 128 wide; d_qk = 192.
//
// Workgroup = (request, head, tile of 32*NW query rows), NW wavefronts of 64
// lanes, one wavefront per 32 query rows. Per 64-key tile:
//   S^T[key][q] = K . Q^T     v_mfma_f32_32x32x16_bf16, A = K from LDS, B = Q
//                             held in VGPRs for the whole kernel.
//   online softmax            lane l owns query row l%32; its 32 scores of a
//                             tile sit in its own accumulators and those of
//                             lane l^32, so a row max/sum is one lane swap.
//   O^T[dv][q] += V^T . P^T   A = V^T read from the row-major V tile with
//                             transposing LDS reads, B = P^T converted in
//                             place from the S^T accumulators.
// K and V tiles go from HBM straight into LDS (global_load_lds, no register
// staging) through two or three LDS stages, so the loads of the next tiles
// run while the current one is computed.
#include "mla_internal.h"

namespace {

// max of a value over lanes l and l ^ 32: v_permlane32_swap exchanges the
// two halves of the wavefront in registers (one lane of each pair ends up
// with its own value in one result and its partner's in the other)
__device__ __forceinline__ float xor32_max(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

constexpr int kTileK = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazy = 8.f;      // log2 headroom of the lazy softmax reference

struct AttnArgs {
  const uint16_t* q; int64_t q_rs; int h_begin; int Hsel;
  const uint16_t* k; int64_t khs;
  const uint16_t* v; int64_t vhs;
  const uint16_t* lat; int64_t ld_lat;
  const int32_t* cu_q; const int32_t* cu_k; const int32_t* row_ids;
  int batch; int n_qt; float scale_log2;
  void* out; int64_t out_rs; float* lse; int64_t lse_rs;
  const float* prev; int64_t prev_rs; const float* prev_lse; int64_t prev_lse_rs;   // merge mode only
  // second key segment (two-segment kernel only): the request's new tokens,
  // causal, with the same latent row stride
  const uint16_t* k2; int64_t khs2; const uint16_t* v2; int64_t vhs2; const uint16_t* lat2;
  const int32_t* cu_k2;
  // two-segment kernel, per request (nullable: every request): nonzero when
  // this pass is the request's last, which takes the second segment and
  // writes the final result to out; the other requests' rows write the
  // running fp32 state to state_out instead
  const int32_t* last; float* state_out; int64_t state_rs;
};

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// LDS tiles are filled by global->LDS DMA (one 16-byte chunk per lane, 64
// consecutive chunks per wavefront instruction), so rows carry no padding;
// bank conflicts of the fragment reads are removed by XOR-swizzling chunk
// positions inside a row instead. Measured on gfx950 with rocprofv3
// (SQ_LDS_BANK_CONFLICT) both read patterns below are conflict-free, while the
// unswizzled layouts cost 4 (K) and 6 (V) conflict cycles per read.
//   K tile: a k_nope region, 64 keys x 256 B (16 chunks), chunk c of key r
//           at position c ^ (r & 15); then a k_rope region, 64 keys x 128 B
//           (8 chunks), chunk c of key r at position c ^ ((r >> 1) & 7).
//           Separate regions let every DMA instruction take one source (the
//           head's k_nope rows or the latent's k_rope columns) as a
//           wavefront-uniform base plus a fixed per-lane offset.
//   V tile: 64 keys x 256 B (16 chunks), row-major; chunk c of key r sits at
//           position c ^ ((r & 3) << 2). The PV operand (eight keys of one dv
//           column per lane) is read with ds_read_b64_tr_b16, which hands
//           each lane four consecutive keys of one column.
constexpr int kKNRow = 256;                // bytes per key in the k_nope region
constexpr int kKRRow = 128;                // bytes per key in the k_rope region
constexpr int kKNope = 64 * kKNRow;        // k_nope region bytes (16384)
constexpr int kVRow = 256;                 // bytes per V row in LDS
constexpr int kKTile = kKNope + 64 * kKRRow;   // 24576
constexpr int kVTile = kTileK * kVRow;     // 16384

constexpr int kStage = kKTile + kVTile;   // one LDS stage: K tile then V tile

// kSeg2: after the keys of cu_k (all visible), the keys of cu_k2 from the
// second segment, causal (row i sees key j iff j <= i + n_k2 - n_q), in the
// same online softmax: the last context chunk and the new tokens in one pass.
template <int NW, bool kCausal, bool kRowIds, int kOutDt, bool kMerge, bool kSeg2 = false>
__global__ __launch_bounds__(NW * 64) void attn_kernel(AttnArgs a) {
  static_assert(!(kSeg2 && (kCausal || kRowIds)), "two segments: plain first segment, no row ids");
  constexpr int ROWS = 32 * NW;
  constexpr int NB = (NW == 8) ? 3 : 2;   // LDS stages (tiles in flight)
  constexpr int kKnj = (kTileK * 16) / (64 * NW);  // k_nope DMA instructions per wavefront per tile
  constexpr int kKrj = (kTileK * 8) / (64 * NW);   // k_rope DMA instructions per wavefront per tile
  constexpr int kKj = kKnj + kKrj;
  constexpr int kVj = (kTileK * 16) / (64 * NW);   // V DMA instructions per wavefront per tile
  constexpr int kDma = kKj + kVj;
  static_assert(kKnj * 64 * NW == kTileK * 16 && kKrj * 64 * NW == kTileK * 8 && kVj * 64 * NW == kTileK * 16,
                "tile split");
  // LDS fragment reads issued ahead of their products (K: of 24 per tile, V:
  // of 32)
  constexpr int kKAhead = 6;
  constexpr int kVAhead = 8;

  // one array per stage (K tile then V tile); two stages take 80 KB, so two
  // 4-wavefront workgroups fit in one CU's 160 KB
  __shared__ __attribute__((aligned(1024))) uint8_t Sm[NB * kStage];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;

  // Workgroups are dispatched round-robin over the 8 XCDs (blockIdx % 8).
  // (request, head) pairs are dealt to the XCDs round-robin too, with all
  // query tiles of one pair on the same XCD, where they share the pair's K
  // and V in L2. Dealing pairs (not contiguous ranges of them) keeps the XCDs
  // evenly loaded when request lengths differ.
  const int n_bh = a.batch * a.Hsel;
  const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
  const int bh = (j / a.n_qt) * 8 + xcd;
  if (bh >= n_bh) return;
  int qt = j % a.n_qt;
  const int hs = bh % a.Hsel;
  const int b = bh / a.Hsel;
  // longest rows first: later row tiles see more keys of a causal segment
  if (kCausal || kSeg2) qt = a.n_qt - 1 - qt;

  const int q0 = a.cu_q[b];
  const int n_q = a.cu_q[b + 1] - q0;
  const int r0 = qt * ROWS;
  if (r0 >= n_q) return;
  const int k0 = a.cu_k[b];
  const int n_k = a.cu_k[b + 1] - k0;
  const int shift = n_k - n_q;               // causal: row i sees key j iff j <= i + shift
  int kend = n_k;
  if (kCausal) kend = min(n_k, r0 + ROWS + shift);
  const int ntiles1 = kend > 0 ? (kend + kTileK - 1) / kTileK : 0;   // tiles of the first segment
  int ntiles = ntiles1;
  int k02 = 0, n_k2 = 0, shift2 = 0;
  bool fin = true;                           // this pass writes the request's final result
  if constexpr (kSeg2) {
    fin = a.last == nullptr || a.last[b] != 0;
    k02 = a.cu_k2[b];
    n_k2 = fin ? a.cu_k2[b + 1] - k02 : 0;
    shift2 = n_k2 - n_q;
    const int kend2 = min(n_k2, r0 + ROWS + shift2);
    ntiles += kend2 > 0 ? (kend2 + kTileK - 1) / kTileK : 0;
  }

  // Merging an empty key set into a state in place leaves the state as it
  // is (the identity of the merge): such a workgroup has nothing to read or
  // write. In a chunk loop over ragged requests this skips every request
  // whose context ended in an earlier chunk.
  if constexpr (kMerge && kOutDt == MLA_DTYPE_FP32) {
    if (ntiles == 0 && a.out == static_cast<const void*>(a.prev) && a.out_rs == a.prev_rs &&
        a.lse == a.prev_lse && a.lse_rs == a.prev_lse_rs)
      return;
  }
  if constexpr (kMerge && kSeg2) {
    // a request whose last pass came earlier: its state is no longer read
    if (!fin && ntiles == 0 && a.state_out == a.prev && a.state_rs == a.prev_rs && a.lse == a.prev_lse &&
        a.lse_rs == a.prev_lse_rs)
      return;
  }

  const int row = r0 + wave * 32 + l32;      // this lane's query row (request-local)
  const bool row_ok = row < n_q;
  const int h = a.h_begin + hs;

  // ---- Q fragments (B operand): lane holds q[row][16 s + 8 g .. +8]
  bf16x8 qf[kDqk / 16];
  {
    const uint16_t* qp = nullptr;
    if (row_ok) {
      const int64_t p = kRowIds ? (int64_t)a.row_ids[q0 + row] : (int64_t)(q0 + row);
      qp = a.q + p * a.q_rs + (int64_t)h * kDqk + g * 8;
    }
#pragma unroll
    for (int s = 0; s < kDqk / 16; ++s) {
      u32x4 u = qp ? *reinterpret_cast<const u32x4*>(qp + s * 16) : u32x4{0u, 0u, 0u, 0u};
      qf[s] = __builtin_bit_cast(bf16x8, u);
    }
  }

  const uint16_t* kbase = a.k + (int64_t)hs * a.khs + (int64_t)k0 * kDnope;
  const uint16_t* vbase = a.v + (int64_t)hs * a.vhs + (int64_t)k0 * kDv;
  const uint16_t* rbase = a.lat + (int64_t)k0 * a.ld_lat + kDc;
  const uint16_t* kbase2 = nullptr;
  const uint16_t* vbase2 = nullptr;
  const uint16_t* rbase2 = nullptr;
  if constexpr (kSeg2) {
    kbase2 = a.k2 + (int64_t)hs * a.khs2 + (int64_t)k02 * kDnope;
    vbase2 = a.v2 + (int64_t)hs * a.vhs2 + (int64_t)k02 * kDv;
    rbase2 = a.lat2 + (int64_t)k02 * a.ld_lat + kDc;
  }

  // DMA sources of this lane. Instruction i of a region fills its 1 KB
  // slice: k_nope rows 4i .. 4i+3 (16 chunks each), k_rope rows 8i .. 8i+7 (8
  // chunks each), v rows 4i .. 4i+3; lane l writes LDS chunk l of the slice
  // and reads the global chunk the swizzle puts there. A source is the tile's
  // k_nope, k_rope or v start (wavefront-uniform) plus a per-lane byte
  // offset fixed for the whole kernel. In the last, partial tile keys at or
  // past n_k are clamped to the last key (masked scores, p = 0 values), so no
  // load needs a predicate.
  auto nrow = [&](int jj) { return (jj * NW + wave) * 4 + (lane >> 4); };
  auto rrow = [&](int jj) { return (jj * NW + wave) * 8 + (lane >> 3); };
  auto noff = [&](int r, int rsrc) { return (uint32_t)(rsrc * kKNRow + (((lane & 15) ^ (r & 15)) << 4)); };
  auto roff = [&](int r, int rsrc) {
    return (uint32_t)(rsrc * (int)a.ld_lat * 2 + (((lane & 7) ^ ((r >> 1) & 7)) << 4));
  };
  auto vofs = [&](int r, int rsrc) { return (uint32_t)(rsrc * kVRow + (((lane & 15) ^ ((r & 3) << 2)) << 4)); };
  uint32_t knoff[kKnj], kroff[kKrj], voffd[kVj];
#pragma unroll
  for (int jj = 0; jj < kKnj; ++jj) knoff[jj] = noff(nrow(jj), nrow(jj));
#pragma unroll
  for (int jj = 0; jj < kKrj; ++jj) kroff[jj] = roff(rrow(jj), rrow(jj));
#pragma unroll
  for (int jj = 0; jj < kVj; ++jj) voffd[jj] = vofs(nrow(jj), nrow(jj));
  // DMA of tile t of the key sequence (the first segment's tiles, then the
  // second's)
  auto dma = [&](uint8_t* St, int t) {
    const bool s2 = kSeg2 && t >= ntiles1;
    const int kt0 = (s2 ? t - ntiles1 : t) * kTileK;
    const int klast = (s2 ? n_k2 : n_k) - 1;
    uint8_t* Kd = St;
    uint8_t* Vd = St + kKTile;
    const uint8_t* nb = reinterpret_cast<const uint8_t*>((s2 ? kbase2 : kbase) + (int64_t)kt0 * kDnope);
    const uint8_t* rb = reinterpret_cast<const uint8_t*>((s2 ? rbase2 : rbase) + (int64_t)kt0 * a.ld_lat);
    const uint8_t* vb = reinterpret_cast<const uint8_t*>((s2 ? vbase2 : vbase) + (int64_t)kt0 * kDv);
    if (kt0 + kTileK - 1 <= klast) {
#pragma unroll
      for (int jj = 0; jj < kKnj; ++jj) dma16s(nb, knoff[jj], Kd + (jj * NW + wave) * 1024);
#pragma unroll
      for (int jj = 0; jj < kKrj; ++jj) dma16s(rb, kroff[jj], Kd + kKNope + (jj * NW + wave) * 1024);
#pragma unroll
      for (int jj = 0; jj < kVj; ++jj) dma16s(vb, voffd[jj], Vd + (jj * NW + wave) * 1024);
    } else {
      // last tile: rows past the last key read the last key
      const int rl = klast - kt0;
#pragma unroll
      for (int jj = 0; jj < kKnj; ++jj)
        dma16s(nb, noff(nrow(jj), min(nrow(jj), rl)), Kd + (jj * NW + wave) * 1024);
#pragma unroll
      for (int jj = 0; jj < kKrj; ++jj)
        dma16s(rb, roff(rrow(jj), min(rrow(jj), rl)), Kd + kKNope + (jj * NW + wave) * 1024);
#pragma unroll
      for (int jj = 0; jj < kVj; ++jj)
        dma16s(vb, vofs(nrow(jj), min(nrow(jj), rl)), Vd + (jj * NW + wave) * 1024);
    }
  };

  // per-lane fragment read offsets (bytes)
  // K: key l32 (+ 32 for the second block, a constant offset), dims
  // 16 s + 8 g .. +8: chunk 2 s + g of the k_nope region for s < 8, chunk
  // 2 (s - 8) + g of the k_rope region for s >= 8
  int koff[kDqk / 16];
#pragma unroll
  for (int s2 = 0; s2 < kDqk / 16; ++s2)
    koff[s2] = s2 < 8 ? l32 * kKNRow + (((2 * s2 + g) ^ (l32 & 15)) << 4)
                      : kKNope + l32 * kKRRow + (((2 * (s2 - 8) + g) ^ ((l32 >> 1) & 7)) << 4);
  int voff[4];                               // V^T: dv block d; + (16 mm + 8 half) rows
  {
    const int a4 = (lane & 15) >> 2, b4 = lane & 3, g16 = (lane >> 4) & 1;
#pragma unroll
    for (int d = 0; d < 4; ++d) voff[d] = (4 * g + a4) * kVRow + 64 * (d ^ a4) + 32 * g16 + 8 * b4;
  }

  f32x16 O[4];
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int i = 0; i < 16; ++i) O[d][i] = 0.f;
  float m_ref = -INFINITY, l_run = 0.f;     // reference max (scaled, log2 units), row sum
  f32x16 S[2];                               // S^T of the current tile
  bf16x8 P[4];                               // P^T operands of the tile being multiplied by V
  bool rescale = false;                      // O needs the factor alpha_o before the next PV
  float alpha_o = 1.f;

  // last key (exclusive) any row of this wavefront may see; a wavefront
  // whose rows all lie past the request's rows (the last row tile of a short
  // request) sees none and only takes part in the DMA and the barriers
  const int wave_kend = (r0 + wave * 32 >= n_q) ? 0
                        : kCausal ? min(n_k, r0 + wave * 32 + 32 + shift) : n_k;
  const int wave_first_lim = r0 + wave * 32 + shift;   // causal: smallest row limit in the wave
  const int row_lim = row + shift;           // causal: keys <= row_lim are visible
  // the same for the second segment
  const int wave_kend2 = (r0 + wave * 32 >= n_q) ? 0 : min(n_k2, r0 + wave * 32 + 32 + shift2);
  const int wave_first_lim2 = r0 + wave * 32 + shift2;
  const int row_lim2 = row + shift2;
  const float c = a.scale_log2;              // scale * log2(e); scores stay raw until exp2

  // S^T = K . Q^T for one tile
  auto qk = [&](const uint8_t* Ks) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) S[kb][i] = 0.f;
#pragma unroll
    for (int s = 0; s < kDqk / 16; ++s) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(Ks + koff[s] + kb * 32 * (s < 8 ? kKNRow : kKRRow));
        S[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], S[kb], 0, 0, 0);
      }
    }
    // keep the K fragment reads kKAhead ahead of the products that use them
    __builtin_amdgcn_sched_group_barrier(0x100, kKAhead, 0);
#pragma unroll
    for (int i = 0; i < (24 - kKAhead) / 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kKAhead, 0);
  };

  // online softmax of the tile in S (keys kt0..kt0+63 of the first
  // segment, or of the second when s2) -> P, rescaling O
  auto softmax = [&](int kt0, bool s2) {
    // masking only on tiles that cross the key end or the causal diagonal
    const bool causal = kCausal || s2;
    const int nk = s2 ? n_k2 : n_k;
    const int first_lim = s2 ? wave_first_lim2 : wave_first_lim;
    const int rlim = s2 ? row_lim2 : row_lim;
    const bool edge = (kt0 + kTileK > nk) || (causal && kt0 + kTileK - 1 > first_lim);
    if (edge) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kt0 + kb * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
          const bool vis = key < nk && (!causal || key <= rlim);
          S[kb][i] = vis ? S[kb][i] : -INFINITY;
        }
    }
    // row max of raw scores (scale > 0 keeps the order): own 32 keys, then lane ^ 32
    float mt = S[0][0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mt = fmaxf(mt, S[0][i]);
#pragma unroll
    for (int i = 0; i < 16; ++i) mt = fmaxf(mt, S[1][i]);
    mt = xor32_max(mt);
    // Lazy reference max (log2 units): it only moves when the tile max
    // exceeds it by more than kLazy, so p <= 2^kLazy and the rescale of O is
    // skipped on almost every tile. The normalisation uses the same
    // reference, so the result does not depend on when it moved.
    const float mtc = mt * c;
    const bool bump = mtc > m_ref + kLazy;     // false while mt = -inf
    const float m_new = bump ? mtc : m_ref;
    const float alpha = bump ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.f;   // 0 from -inf
    const float mc = (m_new == -INFINITY) ? 0.f : m_new;
    float ps = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(fmaf(S[kb][i], c, -mc));
        S[kb][i] = p;
        ps += p;
      }
    l_run = fmaf(l_run, alpha, ps);
    // O is rescaled by alpha right before the next PV products
    rescale = __any(bump);
    alpha_o = alpha;
    m_ref = m_new;
    // P^T operand of MFMA mm (keys 16mm..16mm+15 of the tile): lane slots
    // 0-3 hold keys 16mm+4g+0..3, slots 4-7 keys 16mm+8+4g+0..3, which is
    // where the S^T accumulator layout puts them
#pragma unroll
    for (int mm = 0; mm < 4; ++mm) {
      const int kb = mm >> 1, i0 = 8 * (mm & 1);
      u32x4 u;
      u.x = cvt_pk_bf16(S[kb][i0 + 0], S[kb][i0 + 1]);
      u.y = cvt_pk_bf16(S[kb][i0 + 2], S[kb][i0 + 3]);
      u.z = cvt_pk_bf16(S[kb][i0 + 4], S[kb][i0 + 5]);
      u.w = cvt_pk_bf16(S[kb][i0 + 6], S[kb][i0 + 7]);
      P[mm] = __builtin_bit_cast(bf16x8, u);
    }
  };

  // O^T += V^T . P^T; the V^T operand is read for the P^T keys with two
  // transposing reads
  auto pv = [&](const uint8_t* Vs) {
    if (rescale) {
#pragma unroll
      for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int i = 0; i < 16; ++i) O[d][i] *= alpha_o;
    }
#pragma unroll
    for (int mm = 0; mm < 4; ++mm) {
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint8_t* vp = Vs + voff[d] + 16 * mm * kVRow;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vp));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vp + 8 * kVRow));
        const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        O[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, P[mm], O[d], 0, 0, 0);
      }
    }
    // V reads kVAhead reads ahead of the products
    __builtin_amdgcn_sched_group_barrier(0x100, kVAhead, 1);
#pragma unroll
    for (int i = 0; i < (32 - kVAhead) / 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kVAhead / 2, 1);
  };

  auto stage = [&](int t) -> uint8_t* { return Sm + (t % NB) * kStage; };

  // Pipeline over key tiles with NB LDS stages: step t waits for its own
  // DMA of tile t, meets the others at the barrier (after which tile t is
  // visible and stage (t-1) % NB is free), issues the DMA of tile t+NB-1
  // into that stage and computes tile t. Tile indices past the end are
  // clamped to the last tile, so every step issues the same number of DMA
  // instructions and the vector-memory counter stays exact.
  if (ntiles > 0) {
    dma(stage(0), 0);
    if (NB == 3) dma(stage(1), min(1, ntiles - 1));
  }
  // the Q fragments (and the first tiles) have landed: without this wait
  // the compiler, which does not see the DMA, would wait for every
  // outstanding load before the first product of each tile
  wait_vmcnt<0>();
  for (int kt = 0; kt < ntiles; ++kt) {
    const bool s2 = kSeg2 && kt >= ntiles1;
    const int kt0 = (s2 ? kt - ntiles1 : kt) * kTileK;
    wait_vmcnt<kDma * (NB - 2)>();
    __syncthreads();
    dma(stage(kt + NB - 1), min(kt + NB - 1, ntiles - 1));
    if (kt0 < (s2 ? wave_kend2 : wave_kend)) {
      qk(stage(kt));
      softmax(kt0, s2);
      // The PV products run at raised wave priority: of the two wavefronts
      // a SIMD holds (two workgroups per CU), the one with products ready
      // keeps the matrix core fed while the other computes its softmax.
      __builtin_amdgcn_s_setprio(1);
      pv(stage(kt) + kKTile);
      __builtin_amdgcn_s_setprio(0);
    }
  }
  // no DMA may still be writing this workgroup's LDS when it ends
  wait_vmcnt<0>();

  // ---- epilogue
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (!row_ok) return;
  const bool empty = !(l_tot > 0.f);
  const int64_t orow = (int64_t)(q0 + row);
  // this state: out = O / l_tot, lse (log2 units) = m_ref + log2 l_tot
  float lse2 = empty ? -INFINITY : m_ref + __builtin_amdgcn_logf(l_tot);
  float c_this = empty ? 0.f : 1.f / l_tot;   // factor on O
  float c_prev = 0.f;                         // factor on the previous out
  const float* pp = nullptr;
  if (kMerge) {
    // Log-sum-exp merge with the previous state of this (row, head), as
    // merge_attn_states does, in log2 units: m = max of the two lse, each
    // side weighted by 2^(lse - m); a side at -inf contributes nothing.
    pp = a.prev + orow * a.prev_rs + (int64_t)hs * kDv;
    const float lp2 = a.prev_lse[orow * a.prev_lse_rs + hs] * kLog2e;
    const float m2 = fmaxf(lse2, lp2);
    if (m2 == -INFINITY) {
      c_this = 0.f;
    } else {
      const float wp = (lp2 == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(lp2 - m2);
      const float wt = (lse2 == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(lse2 - m2);
      const float inv_s = 1.f / (wp + wt);
      c_prev = wp * inv_s;
      c_this *= wt * inv_s;
      lse2 = m2 + __builtin_amdgcn_logf(wp + wt);
    }
  }
  // The previous state is read in full before anything is written: out may
  // be that state (in place), so a read after a store of this lane would
  // have to wait for the store, and 16 read/write round trips in a row
  // measured 8% of a merging pass.
  f32x4 prv[16];
  if (kMerge && c_prev != 0.f) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
      prv[i] = *reinterpret_cast<const f32x4*>(pp + (i >> 2) * 32 + 8 * (i & 3) + 4 * g);
  }
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const int dv = d * 32 + 8 * qq + 4 * g;
      float o0 = O[d][4 * qq + 0] * c_this, o1 = O[d][4 * qq + 1] * c_this;
      float o2 = O[d][4 * qq + 2] * c_this, o3 = O[d][4 * qq + 3] * c_this;
      if (kMerge && c_prev != 0.f) {
        const f32x4 pv = prv[4 * d + qq];
        o0 = fmaf(c_prev, pv.x, o0); o1 = fmaf(c_prev, pv.y, o1);
        o2 = fmaf(c_prev, pv.z, o2); o3 = fmaf(c_prev, pv.w, o3);
      }
      if (kSeg2 && !fin) {
        // not this request's last pass: the running fp32 state
        float* op = a.state_out + orow * a.state_rs + (int64_t)hs * kDv + dv;
        *reinterpret_cast<f32x4*>(op) = f32x4{o0, o1, o2, o3};
      } else if (kOutDt == MLA_DTYPE_FP32) {
        float* op = static_cast<float*>(a.out) + orow * a.out_rs + (int64_t)hs * kDv + dv;
        *reinterpret_cast<f32x4*>(op) = f32x4{o0, o1, o2, o3};
      } else {
        uint16_t* op = static_cast<uint16_t*>(a.out) + orow * a.out_rs + (int64_t)hs * kDv + dv;
        *reinterpret_cast<u32x2*>(op) = u32x2{cvt_pk_bf16(o0, o1), cvt_pk_bf16(o2, o3)};
      }
    }
  if (g == 0) a.lse[orow * a.lse_rs + hs] = lse2 * kLn2;
}

template <int NW, bool kMerge>
void launch_seg2(int out_dt, dim3 g, hipStream_t s, const AttnArgs& a) {
  if (out_dt == MLA_DTYPE_FP32)
    hipLaunchKernelGGL((attn_kernel<NW, false, false, MLA_DTYPE_FP32, kMerge, true>), g, dim3(NW * 64), 0, s, a);
  else
    hipLaunchKernelGGL((attn_kernel<NW, false, false, MLA_DTYPE_BF16, kMerge, true>), g, dim3(NW * 64), 0, s, a);
}
template <int NW>
void launch_seg2m(bool merge, int out_dt, dim3 g, hipStream_t s, const AttnArgs& a) {
  if (merge) launch_seg2<NW, true>(out_dt, g, s, a);
  else launch_seg2<NW, false>(out_dt, g, s, a);
}

// second key segment of mla_prefill_attn_2seg and mla_prefill_attn_chunk;
// the latter also passes the per-request last-pass flags and the fp32 state
// the other requests' rows write
struct Seg2 {
  const void* k_nope; int64_t k_head_stride; const void* v; int64_t v_head_stride;
  const void* latent; int64_t ld_latent; const int32_t* cu_k;
  const int32_t* last = nullptr; float* state = nullptr; int64_t state_rs = 0;
};

template <int NW, bool kCausal, bool kRowIds, bool kMerge>
void launch4(int out_dt, dim3 g, hipStream_t s, const AttnArgs& a) {
  if (out_dt == MLA_DTYPE_FP32)
    hipLaunchKernelGGL((attn_kernel<NW, kCausal, kRowIds, MLA_DTYPE_FP32, kMerge>), g, dim3(NW * 64), 0, s, a);
  else
    hipLaunchKernelGGL((attn_kernel<NW, kCausal, kRowIds, MLA_DTYPE_BF16, kMerge>), g, dim3(NW * 64), 0, s, a);
}
template <int NW, bool kCausal, bool kRowIds>
void launch3(bool merge, int out_dt, dim3 g, hipStream_t s, const AttnArgs& a) {
  if (merge) launch4<NW, kCausal, kRowIds, true>(out_dt, g, s, a);
  else launch4<NW, kCausal, kRowIds, false>(out_dt, g, s, a);
}
template <int NW, bool kCausal>
void launch2(bool rowids, bool merge, int out_dt, dim3 g, hipStream_t s, const AttnArgs& a) {
  if (rowids) launch3<NW, kCausal, true>(merge, out_dt, g, s, a);
  else launch3<NW, kCausal, false>(merge, out_dt, g, s, a);
}
template <int NW>
void launch1(bool causal, bool rowids, bool merge, int out_dt, dim3 g, hipStream_t s, const AttnArgs& a) {
  if (causal) launch2<NW, true>(rowids, merge, out_dt, g, s, a);
  else launch2<NW, false>(rowids, merge, out_dt, g, s, a);
}

// validation and launch shared by mla_prefill_attn and mla_prefill_attn_merge
int prefill_attn(const char* fn, const void* q, int64_t q_row_stride, int H_q, int h_begin, int h_end,
                 const void* k_nope, int64_t k_head_stride, const void* v, int64_t v_head_stride,
                 const void* latent, int64_t ld_latent, const int32_t* cu_q, const int32_t* cu_k,
                 const int32_t* q_row_ids, int batch, int max_q, float scale, int causal, void* out,
                 int out_dtype, int64_t out_row_stride, float* lse, int64_t lse_row_stride,
                 const float* prev, int64_t prev_row_stride, const float* prev_lse, int64_t prev_lse_row_stride,
                 bool merge, void* stream, const Seg2* seg2 = nullptr) {
  mla_begin_call();
  MLA_REQUIRE(batch >= 0 && max_q >= 0, MLA_ERR_INVALID_ARG, "%s: batch and max_q must be >= 0", fn);
  MLA_REQUIRE(H_q > 0 && 0 <= h_begin && h_begin < h_end && h_end <= H_q, MLA_ERR_INVALID_ARG,
              "%s: need 0 <= h_begin (%d) < h_end (%d) <= H_q (%d)", fn, h_begin, h_end, H_q);
  if (batch == 0 || max_q == 0) return MLA_OK;
  MLA_REQUIRE(q && k_nope && v && latent && cu_q && cu_k && out && lse, MLA_ERR_INVALID_ARG,
              "%s: null pointer argument", fn);
  MLA_REQUIRE(out_dtype == MLA_DTYPE_BF16 || out_dtype == MLA_DTYPE_FP32, MLA_ERR_UNSUPPORTED,
              "%s: out dtype %d not supported", fn, out_dtype);
  MLA_REQUIRE(mla_aligned16(q) && mla_aligned16(k_nope) && mla_aligned16(v) && mla_aligned16(latent) &&
                  mla_aligned16(out),
              MLA_ERR_INVALID_ARG, "%s: tensor pointers must be 16-byte aligned", fn);
  MLA_REQUIRE(q_row_stride % 8 == 0 && q_row_stride >= (int64_t)H_q * kDqk, MLA_ERR_INVALID_ARG,
              "%s: q_row_stride (%lld) must be a multiple of 8 and >= H_q*192", fn, (long long)q_row_stride);
  MLA_REQUIRE(ld_latent % 8 == 0 && ld_latent >= kDlat && ld_latent <= (1 << 17), MLA_ERR_INVALID_ARG,
              "%s: ld_latent (%lld) must be a multiple of 8 in [576, 2^17]", fn, (long long)ld_latent);
  MLA_REQUIRE(k_head_stride % 8 == 0 && v_head_stride % 8 == 0, MLA_ERR_INVALID_ARG,
              "%s: head strides must be multiples of 8", fn);
  const int Hsel = h_end - h_begin;
  MLA_REQUIRE(out_row_stride % 4 == 0 && out_row_stride >= (int64_t)Hsel * kDv && lse_row_stride >= Hsel,
              MLA_ERR_INVALID_ARG, "%s: out_row_stride must be >= Hsel*128 (multiple of 4), lse_row_stride >= Hsel", fn);
  MLA_REQUIRE(scale > 0.f && scale < 1e30f, MLA_ERR_INVALID_ARG, "%s: scale must be positive and finite", fn);
  if (seg2) {
    MLA_REQUIRE(!causal && !q_row_ids, MLA_ERR_UNSUPPORTED, "%s: the first segment is plain (no causal, no row ids)", fn);
    MLA_REQUIRE(seg2->k_nope && seg2->v && seg2->latent && seg2->cu_k, MLA_ERR_INVALID_ARG,
                "%s: null second-segment argument", fn);
    MLA_REQUIRE(mla_aligned16(seg2->k_nope) && mla_aligned16(seg2->v) && mla_aligned16(seg2->latent),
                MLA_ERR_INVALID_ARG, "%s: second-segment pointers must be 16-byte aligned", fn);
    MLA_REQUIRE(seg2->k_head_stride % 8 == 0 && seg2->v_head_stride % 8 == 0, MLA_ERR_INVALID_ARG,
                "%s: second-segment head strides must be multiples of 8", fn);
    MLA_REQUIRE(seg2->ld_latent == ld_latent, MLA_ERR_UNSUPPORTED,
                "%s: both segments' latents need the same row stride (%lld != %lld)", fn,
                (long long)seg2->ld_latent, (long long)ld_latent);
    if (seg2->last) {
      MLA_REQUIRE(seg2->state, MLA_ERR_INVALID_ARG, "%s: null state", fn);
      MLA_REQUIRE(mla_aligned16(seg2->state) && seg2->state_rs % 4 == 0 && seg2->state_rs >= (int64_t)Hsel * kDv,
                  MLA_ERR_INVALID_ARG, "%s: state must be 16-byte aligned with row stride >= Hsel*128 (multiple of 4)",
                  fn);
    }
  }
  if (merge) {
    MLA_REQUIRE(prev && prev_lse, MLA_ERR_INVALID_ARG, "%s: null previous state", fn);
    MLA_REQUIRE(mla_aligned16(prev) && prev_row_stride % 4 == 0 && prev_row_stride >= (int64_t)Hsel * kDv &&
                    prev_lse_row_stride >= Hsel,
                MLA_ERR_INVALID_ARG,
                "%s: previous state must be 16-byte aligned with row stride >= Hsel*128 (multiple of 4)", fn);
  }

  // rows per workgroup: 128 (4 wavefronts; two workgroups share a CU, 80 KB
  // of two-stage LDS each) by default. Ragged query sets fill 128-row tiles
  // better than 256-row ones, and in a causal segment fewer wavefronts idle
  // above the diagonal. Launches with row ids repeat one full query set for
  // every key piece, so their tiles are never ragged: above 128 rows they use
  // 8 wavefronts (256 rows), which halves the K/V tile loads per row. 64 rows
  // (2 wavefronts) when no request has more.
  int NW = 4;
  if (max_q <= 64) NW = 2;
  else if (q_row_ids != nullptr && max_q > 128 && !causal) NW = 8;
  const int rows = 32 * NW;
  const int n_qt = (max_q + rows - 1) / rows;
  // (request, head) pairs rounded up to a multiple of the 8 XCDs (the
  // surplus workgroups exit at once)
  const int64_t total = ((int64_t)batch * Hsel + 7) / 8 * 8 * n_qt;
  MLA_REQUIRE(total < (int64_t)1 << 31, MLA_ERR_INVALID_ARG, "%s: problem too large", fn);
  AttnArgs a{static_cast<const uint16_t*>(q), q_row_stride, h_begin, Hsel,
             static_cast<const uint16_t*>(k_nope), k_head_stride,
             static_cast<const uint16_t*>(v), v_head_stride,
             static_cast<const uint16_t*>(latent), ld_latent,
             cu_q, cu_k, q_row_ids, batch, n_qt, scale * kLog2e,
             out, out_row_stride, lse, lse_row_stride,
             prev, prev_row_stride, prev_lse, prev_lse_row_stride,
             nullptr, 0, nullptr, 0, nullptr, nullptr, nullptr, nullptr, 0};
  if (seg2) {
    a.k2 = static_cast<const uint16_t*>(seg2->k_nope);
    a.khs2 = seg2->k_head_stride;
    a.v2 = static_cast<const uint16_t*>(seg2->v);
    a.vhs2 = seg2->v_head_stride;
    a.lat2 = static_cast<const uint16_t*>(seg2->latent);
    a.cu_k2 = seg2->cu_k;
    a.last = seg2->last;
    a.state_out = seg2->state;
    a.state_rs = seg2->state_rs;
  }
  dim3 g((unsigned)total);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const bool rid = q_row_ids != nullptr, c = causal != 0;
  if (seg2) {
    if (NW == 4) launch_seg2m<4>(merge, out_dtype, g, s, a);   // no row ids: never 8 wavefronts
    else launch_seg2m<2>(merge, out_dtype, g, s, a);
    return mla_check_launch(fn);
  }
  if (NW == 8) launch1<8>(c, rid, merge, out_dtype, g, s, a);
  else if (NW == 4) launch1<4>(c, rid, merge, out_dtype, g, s, a);
  else launch1<2>(c, rid, merge, out_dtype, g, s, a);
  return mla_check_launch(fn);
}

}  // namespace

extern "C" int mla_prefill_attn(const void* q, int64_t q_row_stride, int H_q, int h_begin, int h_end,
                                const void* k_nope, int64_t k_head_stride,
                                const void* v, int64_t v_head_stride,
                                const void* latent, int64_t ld_latent,
                                const int32_t* cu_q, const int32_t* cu_k, const int32_t* q_row_ids,
                                int batch, int max_q, float scale, int causal,
                                void* out, int out_dtype, int64_t out_row_stride,
                                float* lse, int64_t lse_row_stride, void* stream) {
  return prefill_attn("mla_prefill_attn", q, q_row_stride, H_q, h_begin, h_end, k_nope, k_head_stride, v,
                      v_head_stride, latent, ld_latent, cu_q, cu_k, q_row_ids, batch, max_q, scale, causal,
                      out, out_dtype, out_row_stride, lse, lse_row_stride, nullptr, 0, nullptr, 0, false, stream);
}

extern "C" int mla_prefill_attn_merge(const void* q, int64_t q_row_stride, int H_q, int h_begin, int h_end,
                                      const void* k_nope, int64_t k_head_stride,
                                      const void* v, int64_t v_head_stride,
                                      const void* latent, int64_t ld_latent,
                                      const int32_t* cu_q, const int32_t* cu_k, const int32_t* q_row_ids,
                                      int batch, int max_q, float scale, int causal,
                                      const float* prev_out, int64_t prev_row_stride,
                                      const float* prev_lse, int64_t prev_lse_row_stride,
                                      void* out, int out_dtype, int64_t out_row_stride,
                                      float* lse, int64_t lse_row_stride, void* stream) {
  return prefill_attn("mla_prefill_attn_merge", q, q_row_stride, H_q, h_begin, h_end, k_nope, k_head_stride,
                      v, v_head_stride, latent, ld_latent, cu_q, cu_k, q_row_ids, batch, max_q, scale, causal,
                      out, out_dtype, out_row_stride, lse, lse_row_stride, prev_out, prev_row_stride, prev_lse,
                      prev_lse_row_stride, true, stream);
}

extern "C" int mla_prefill_attn_2seg(const void* q, int64_t q_row_stride, int H_q, int h_begin, int h_end,
                                     const void* k_nope, int64_t k_head_stride, const void* v,
                                     int64_t v_head_stride, const void* latent, int64_t ld_latent,
                                     const int32_t* cu_k, const void* k_nope2, int64_t k_head_stride2,
                                     const void* v2, int64_t v_head_stride2, const void* latent2,
                                     int64_t ld_latent2, const int32_t* cu_k2, const int32_t* cu_q, int batch,
                                     int max_q, float scale, const float* prev_out, int64_t prev_row_stride,
                                     const float* prev_lse, int64_t prev_lse_row_stride, void* out,
                                     int out_dtype, int64_t out_row_stride, float* lse, int64_t lse_row_stride,
                                     void* stream) {
  const Seg2 seg2{k_nope2, k_head_stride2, v2, v_head_stride2, latent2, ld_latent2, cu_k2};
  const bool merge = prev_out != nullptr || prev_lse != nullptr;
  return prefill_attn("mla_prefill_attn_2seg", q, q_row_stride, H_q, h_begin, h_end, k_nope, k_head_stride, v,
                      v_head_stride, latent, ld_latent, cu_q, cu_k, nullptr, batch, max_q, scale, 0, out,
                      out_dtype, out_row_stride, lse, lse_row_stride, prev_out, prev_row_stride, prev_lse,
                      prev_lse_row_stride, merge, stream, &seg2);
}

extern "C" int mla_prefill_attn_chunk(const void* q, int64_t q_row_stride, int H_q, int h_begin, int h_end,
                                      const void* k_nope, int64_t k_head_stride, const void* v,
                                      int64_t v_head_stride, const void* latent, int64_t ld_latent,
                                      const int32_t* cu_k, const void* k_nope2, int64_t k_head_stride2,
                                      const void* v2, int64_t v_head_stride2, const void* latent2,
                                      int64_t ld_latent2, const int32_t* cu_k2, const int32_t* last,
                                      const int32_t* cu_q, int batch, int max_q, float scale, int merge,
                                      float* state, int64_t state_row_stride, float* state_lse,
                                      int64_t state_lse_row_stride, void* out, int64_t out_row_stride,
                                      void* stream) {
  const char* fn = "mla_prefill_attn_chunk";
  if (batch > 0 && max_q > 0 && !(last && state && state_lse)) {
    mla_begin_call();
    mla_set_error("%s: null last, state or state_lse", fn);
    return MLA_ERR_INVALID_ARG;
  }
  Seg2 seg2{k_nope2, k_head_stride2, v2, v_head_stride2, latent2, ld_latent2, cu_k2};
  seg2.last = last;
  seg2.state = state;
  seg2.state_rs = state_row_stride;
  return prefill_attn(fn, q, q_row_stride, H_q, h_begin, h_end, k_nope, k_head_stride, v, v_head_stride, latent,
                      ld_latent, cu_q, cu_k, nullptr, batch, max_q, scale, 0, out, MLA_DTYPE_BF16, out_row_stride,
                      state_lse, state_lse_row_stride, merge ? state : nullptr, state_row_stride,
                      merge ? state_lse : nullptr, state_lse_row_stride, merge != 0, stream, &seg2);
}
