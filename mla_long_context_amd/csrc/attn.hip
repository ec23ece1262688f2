// Flash-attention prefill returning (out, lse) for MLA on gfx950: the context
// pass (no mask) and the causal extend pass of the two-stage prefill
// (DeepSeek MLA -- Prefix Cache and Chunked Prefill, sections 4.2 and 4.4
// steps 3-4). Keys are K = [k_nope (per head, 128) | k_rope (64, one per token,
// shared by every head)]; values are per head, 128 wide; d_qk = 192.
//
// Workgroup = (request, head, tile of 32*NW query rows), NW wavefronts of 64
// lanes, one wavefront per 32 query rows. Per 64-key tile:
//   S^T[key][q] = K . Q^T     v_mfma_f32_32x32x16_bf16, A = K from LDS (the
//                             k_rope columns are read once per tile for the
//                             workgroup), B = Q held in VGPRs for the kernel.
//   online softmax            lane l owns query row l%32; its 32 scores of a
//                             tile sit in its own accumulators and those of
//                             lane l^32, so a row max/sum is one lane swap.
//   O^T[dv][q] += V^T . P^T   A = V^T from LDS, B = P^T converted in place
//                             from the S^T accumulators (no LDS round trip).
// V rows are transposed into LDS with a 4x4 register transpose, and the key
// order inside each 16-key group is permuted so that the PV operand of a
// lane is one 16-byte LDS read. The next tile is prefetched into registers
// while the current one is consumed.
#include "mla_internal.h"

namespace {

constexpr int kTileK = 64;
constexpr int kKsLd = kDqk + 8;   // 200 elements = 400 B per key row (conflict-free b128 reads)
constexpr int kVtLd = kTileK + 8; // 72 elements = 144 B per dv row
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
};

// V^T tile in LDS: row = dv (0..127), 64 key positions per row, 144-byte row
// pitch. On gfx950 (128 LDS banks, 16-byte reads served 32 lanes at a time)
// this pitch makes the fragment reads conflict-free, and the transpose writes
// are conflict-free when the 16 key quads of a tile vary fastest across lanes
// (lane -> (kq = idx & 15, dq = idx >> 4)); with dv quads fastest instead,
// rocprofv3 counted 28 bank-conflict cycles per write instruction.
__device__ __forceinline__ int vt_index(int row, int pos) { return row * kVtLd + pos; }

__device__ __forceinline__ int perm_quad(int kq) {
  // key quad kq (0..15 in the tile) -> LDS position of its 4 keys
  const int q4 = kq & 3;
  const int pos4 = (q4 == 1) ? 2 : (q4 == 2 ? 1 : q4);
  return (kq & ~3) * 4 + pos4 * 4;
}

template <int NW, bool kCausal, bool kRowIds, int kOutDt>
__global__ __launch_bounds__(NW * 64) void attn_kernel(AttnArgs a) {
  constexpr int NT = NW * 64;
  constexpr int ROWS = 32 * NW;
  constexpr int kKv = (kTileK * 16) / NT;    // 16-byte k_nope vectors per thread
  constexpr int kRv = (kTileK * 8) / NT;     // 16-byte rope vectors per thread (>= 1 for NW <= 8)
  constexpr int kVb = (16 * 32) / NT;        // 4x4 V blocks per thread
  static_assert(kKv >= 1 && kRv >= 1 && kVb >= 1, "tile split");

  // two LDS buffers: tile t is consumed from one while tile t+1 is written
  // into the other, so one barrier per tile suffices
  __shared__ __attribute__((aligned(16))) uint16_t Ks2[2][kTileK * kKsLd];
  __shared__ __attribute__((aligned(16))) uint16_t Vt2[2][kDv * kVtLd];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;

  const uint32_t total = (uint32_t)a.batch * a.Hsel * a.n_qt;
  const uint32_t w = xcd_remap(blockIdx.x, total);
  int qt = (int)(w % (uint32_t)a.n_qt);
  const int hs = (int)((w / (uint32_t)a.n_qt) % (uint32_t)a.Hsel);
  const int b = (int)(w / ((uint32_t)a.n_qt * a.Hsel));
  if (kCausal) qt = a.n_qt - 1 - qt;   // longest rows first

  const int q0 = a.cu_q[b];
  const int n_q = a.cu_q[b + 1] - q0;
  const int r0 = qt * ROWS;
  if (r0 >= n_q) return;
  const int k0 = a.cu_k[b];
  const int n_k = a.cu_k[b + 1] - k0;
  const int shift = n_k - n_q;               // causal: row i sees key j iff j <= i + shift
  int kend = n_k;
  if (kCausal) kend = min(n_k, r0 + ROWS + shift);
  const int ntiles = kend > 0 ? (kend + kTileK - 1) / kTileK : 0;

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

  // register prefetch buffers: two tiles in flight (tile t+2 is loaded while
  // tile t is computed and tile t+1 is written to LDS)
  struct Pref {
    u32x4 k[kKv], r[kRv];
    u32x2 v[kVb][4];
  };
  Pref pa, pb;
  // Keys at or past n_k are clamped to the last key: their scores are masked
  // to -inf and their values meet p = 0, so no load needs a predicate.
  const int klast = n_k - 1;
  auto gload = [&](Pref& pf, int kt0) {
#pragma unroll
    for (int j = 0; j < kKv; ++j) {
      const int idx = tid + NT * j, key = min(kt0 + (idx >> 4), klast), vec = idx & 15;
      pf.k[j] = *reinterpret_cast<const u32x4*>(kbase + key * kDnope + vec * 8);
    }
#pragma unroll
    for (int j = 0; j < kRv; ++j) {
      const int idx = tid + NT * j, key = min(kt0 + (idx >> 3), klast), vec = idx & 7;
      pf.r[j] = *reinterpret_cast<const u32x4*>(rbase + (int64_t)key * a.ld_lat + vec * 8);
    }
#pragma unroll
    for (int j = 0; j < kVb; ++j) {
      const int idx = tid + NT * j, kq = idx & 15, dq = idx >> 4;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = min(kt0 + kq * 4 + r, klast);
        pf.v[j][r] = *reinterpret_cast<const u32x2*>(vbase + key * kDv + dq * 4);
      }
    }
  };
  auto lstore = [&](const Pref& pf, int buf) {
    uint16_t* Ks = Ks2[buf];
    uint16_t* Vt = Vt2[buf];
#pragma unroll
    for (int j = 0; j < kKv; ++j) {
      const int idx = tid + NT * j, key = idx >> 4, vec = idx & 15;
      *reinterpret_cast<u32x4*>(Ks + key * kKsLd + vec * 8) = pf.k[j];
    }
#pragma unroll
    for (int j = 0; j < kRv; ++j) {
      const int idx = tid + NT * j, key = idx >> 3, vec = idx & 7;
      *reinterpret_cast<u32x4*>(Ks + key * kKsLd + kDnope + vec * 8) = pf.r[j];
    }
#pragma unroll
    for (int j = 0; j < kVb; ++j) {
      const int idx = tid + NT * j, kq = idx & 15, dq = idx >> 4;
      const int pos = perm_quad(kq);
      // 4x4 transpose of bf16: rows = keys r, cols = dv c
      const uint32_t x0 = pf.v[j][0].x, y0 = pf.v[j][0].y, x1 = pf.v[j][1].x, y1 = pf.v[j][1].y;
      const uint32_t x2 = pf.v[j][2].x, y2 = pf.v[j][2].y, x3 = pf.v[j][3].x, y3 = pf.v[j][3].y;
      u32x2 c0 = {(x0 & 0xffffu) | (x1 << 16), (x2 & 0xffffu) | (x3 << 16)};
      u32x2 c1 = {(x0 >> 16) | (x1 & 0xffff0000u), (x2 >> 16) | (x3 & 0xffff0000u)};
      u32x2 c2 = {(y0 & 0xffffu) | (y1 << 16), (y2 & 0xffffu) | (y3 << 16)};
      u32x2 c3 = {(y0 >> 16) | (y1 & 0xffff0000u), (y2 >> 16) | (y3 & 0xffff0000u)};
      *reinterpret_cast<u32x2*>(Vt + vt_index(dq * 4 + 0, pos)) = c0;
      *reinterpret_cast<u32x2*>(Vt + vt_index(dq * 4 + 1, pos)) = c1;
      *reinterpret_cast<u32x2*>(Vt + vt_index(dq * 4 + 2, pos)) = c2;
      *reinterpret_cast<u32x2*>(Vt + vt_index(dq * 4 + 3, pos)) = c3;
    }
  };

  f32x16 O[4];
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int i = 0; i < 16; ++i) O[d][i] = 0.f;
  float m_ref = -INFINITY, l_run = 0.f;     // reference max (scaled, log2 units), row sum

  // last key (exclusive) any row of this wavefront may see
  const int wave_kend = kCausal ? min(n_k, r0 + wave * 32 + 32 + shift) : n_k;
  const int wave_first_lim = r0 + wave * 32 + shift;   // causal: smallest row limit in the wave
  const int row_lim = row + shift;           // causal: keys <= row_lim are visible
  const float c = a.scale_log2;              // scale * log2(e); scores stay raw until exp2

  // software pipeline over key tiles: iteration t loads tile t+2 into one
  // register buffer, computes tile t from LDS buffer t%2, and writes tile t+1
  // (loaded one iteration earlier) into LDS buffer (t+1)%2. Out-of-range tile
  // indices are clamped to the last tile: harmless re-reads keep the loop
  // body branch-free.
  const int last_kt0 = (ntiles - 1) * kTileK;
  if (ntiles > 0) {
    gload(pa, 0);
    gload(pb, min(kTileK, last_kt0));
    lstore(pa, 0);
  }
  __syncthreads();
  // pn: free register buffer (its tile is already in LDS); pw: holds tile t+1
  auto step = [&](int kt, Pref& pn, Pref& pw) {
    const int kt0 = kt * kTileK;
    const int cur = kt & 1;
    gload(pn, min(kt0 + 2 * kTileK, last_kt0));
    __builtin_amdgcn_sched_barrier(0);
    const uint16_t* Ks = Ks2[cur];
    const uint16_t* Vt = Vt2[cur];
    if (kt0 < wave_kend) {
      f32x16 S[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) S[kb][i] = 0.f;
#pragma unroll
      for (int s = 0; s < kDqk / 16; ++s) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const bf16x8 kf = *reinterpret_cast<const bf16x8*>(Ks + (kb * 32 + l32) * kKsLd + s * 16 + g * 8);
          S[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], S[kb], 0, 0, 0);
        }
      }
      // masking only on tiles that cross the key end or the causal diagonal
      const bool edge = (kt0 + kTileK > n_k) || (kCausal && kt0 + kTileK - 1 > wave_first_lim);
      if (edge) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = kt0 + kb * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
            const bool vis = key < n_k && (!kCausal || key <= row_lim);
            S[kb][i] = vis ? S[kb][i] : -INFINITY;
          }
      }
      // row max of raw scores (scale > 0 keeps the order): own 32 keys, then lane ^ 32
      float mt = S[0][0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mt = fmaxf(mt, S[0][i]);
#pragma unroll
      for (int i = 0; i < 16; ++i) mt = fmaxf(mt, S[1][i]);
      mt = fmaxf(mt, __shfl_xor(mt, 32));
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
      if (__any(bump)) {
#pragma unroll
        for (int d = 0; d < 4; ++d)
#pragma unroll
          for (int i = 0; i < 16; ++i) O[d][i] *= alpha;
      }
      m_ref = m_new;
      // P^T operands: MFMA mm covers keys 16mm..16mm+15 of the tile
#pragma unroll
      for (int mm = 0; mm < 4; ++mm) {
        const int kb = mm >> 1, i0 = 8 * (mm & 1);
        u32x4 u;
        u.x = cvt_pk_bf16(S[kb][i0 + 0], S[kb][i0 + 1]);
        u.y = cvt_pk_bf16(S[kb][i0 + 2], S[kb][i0 + 3]);
        u.z = cvt_pk_bf16(S[kb][i0 + 4], S[kb][i0 + 5]);
        u.w = cvt_pk_bf16(S[kb][i0 + 6], S[kb][i0 + 7]);
        const bf16x8 pf = __builtin_bit_cast(bf16x8, u);
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const bf16x8 vf = *reinterpret_cast<const bf16x8*>(Vt + vt_index(d * 32 + l32, mm * 16 + g * 8));
          O[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, O[d], 0, 0, 0);
        }
      }
    }
    lstore(pw, cur ^ 1);
    __syncthreads();
  };
  // unrolled by two so each register buffer keeps fixed registers
  for (int kt = 0; kt < ntiles; kt += 2) {
    step(kt, pa, pb);
    if (kt + 1 < ntiles) step(kt + 1, pb, pa);
  }


  // ---- epilogue
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (!row_ok) return;
  const bool empty = !(l_tot > 0.f);
  const float inv = empty ? 0.f : 1.f / l_tot;
  const int64_t orow = (int64_t)(q0 + row);
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const int dv = d * 32 + 8 * qq + 4 * g;
      const float o0 = O[d][4 * qq + 0] * inv, o1 = O[d][4 * qq + 1] * inv;
      const float o2 = O[d][4 * qq + 2] * inv, o3 = O[d][4 * qq + 3] * inv;
      if (kOutDt == MLA_DTYPE_FP32) {
        float* op = static_cast<float*>(a.out) + orow * a.out_rs + (int64_t)hs * kDv + dv;
        *reinterpret_cast<f32x4*>(op) = f32x4{o0, o1, o2, o3};
      } else {
        uint16_t* op = static_cast<uint16_t*>(a.out) + orow * a.out_rs + (int64_t)hs * kDv + dv;
        *reinterpret_cast<u32x2*>(op) = u32x2{cvt_pk_bf16(o0, o1), cvt_pk_bf16(o2, o3)};
      }
    }
  if (g == 0)
    a.lse[orow * a.lse_rs + hs] = empty ? -INFINITY : (m_ref + __builtin_amdgcn_logf(l_tot)) * kLn2;
}

template <int NW, bool kCausal, bool kRowIds>
void launch3(int out_dt, dim3 g, hipStream_t s, const AttnArgs& a) {
  if (out_dt == MLA_DTYPE_FP32)
    hipLaunchKernelGGL((attn_kernel<NW, kCausal, kRowIds, MLA_DTYPE_FP32>), g, dim3(NW * 64), 0, s, a);
  else
    hipLaunchKernelGGL((attn_kernel<NW, kCausal, kRowIds, MLA_DTYPE_BF16>), g, dim3(NW * 64), 0, s, a);
}
template <int NW, bool kCausal>
void launch2(bool rowids, int out_dt, dim3 g, hipStream_t s, const AttnArgs& a) {
  if (rowids) launch3<NW, kCausal, true>(out_dt, g, s, a);
  else launch3<NW, kCausal, false>(out_dt, g, s, a);
}
template <int NW>
void launch1(bool causal, bool rowids, int out_dt, dim3 g, hipStream_t s, const AttnArgs& a) {
  if (causal) launch2<NW, true>(rowids, out_dt, g, s, a);
  else launch2<NW, false>(rowids, out_dt, g, s, a);
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
  mla_clear_error();
  MLA_REQUIRE(batch >= 0 && max_q >= 0, MLA_ERR_INVALID_ARG, "mla_prefill_attn: batch and max_q must be >= 0");
  MLA_REQUIRE(H_q > 0 && 0 <= h_begin && h_begin < h_end && h_end <= H_q, MLA_ERR_INVALID_ARG,
              "mla_prefill_attn: need 0 <= h_begin (%d) < h_end (%d) <= H_q (%d)", h_begin, h_end, H_q);
  if (batch == 0 || max_q == 0) return MLA_OK;
  MLA_REQUIRE(q && k_nope && v && latent && cu_q && cu_k && out && lse, MLA_ERR_INVALID_ARG,
              "mla_prefill_attn: null pointer argument");
  MLA_REQUIRE(out_dtype == MLA_DTYPE_BF16 || out_dtype == MLA_DTYPE_FP32, MLA_ERR_UNSUPPORTED,
              "mla_prefill_attn: out dtype %d not supported", out_dtype);
  MLA_REQUIRE(mla_aligned16(q) && mla_aligned16(k_nope) && mla_aligned16(v) && mla_aligned16(latent) &&
                  mla_aligned16(out),
              MLA_ERR_INVALID_ARG, "mla_prefill_attn: tensor pointers must be 16-byte aligned");
  MLA_REQUIRE(q_row_stride % 8 == 0 && q_row_stride >= (int64_t)H_q * kDqk, MLA_ERR_INVALID_ARG,
              "mla_prefill_attn: q_row_stride (%lld) must be a multiple of 8 and >= H_q*192", (long long)q_row_stride);
  MLA_REQUIRE(ld_latent % 8 == 0 && ld_latent >= kDlat, MLA_ERR_INVALID_ARG,
              "mla_prefill_attn: ld_latent (%lld) must be a multiple of 8 and >= 576", (long long)ld_latent);
  MLA_REQUIRE(k_head_stride % 8 == 0 && v_head_stride % 8 == 0, MLA_ERR_INVALID_ARG,
              "mla_prefill_attn: head strides must be multiples of 8");
  const int Hsel = h_end - h_begin;
  MLA_REQUIRE(out_row_stride % 4 == 0 && out_row_stride >= (int64_t)Hsel * kDv && lse_row_stride >= Hsel,
              MLA_ERR_INVALID_ARG, "mla_prefill_attn: out_row_stride must be >= Hsel*128 (multiple of 4), lse_row_stride >= Hsel");
  MLA_REQUIRE(scale > 0.f && scale < 1e30f, MLA_ERR_INVALID_ARG, "mla_prefill_attn: scale must be positive and finite");

  // rows per workgroup: 256 (8 wavefronts) for long query sets, fewer when
  // that would leave most wavefronts without rows or the grid too small.
  int NW = 8;
  if (max_q <= 64) NW = 2;
  else if (max_q <= 128) NW = 4;
  const int rows = 32 * NW;
  const int n_qt = (max_q + rows - 1) / rows;
  const int64_t total = (int64_t)batch * Hsel * n_qt;
  MLA_REQUIRE(total < (int64_t)1 << 31, MLA_ERR_INVALID_ARG, "mla_prefill_attn: problem too large");
  AttnArgs a{static_cast<const uint16_t*>(q), q_row_stride, h_begin, Hsel,
             static_cast<const uint16_t*>(k_nope), k_head_stride,
             static_cast<const uint16_t*>(v), v_head_stride,
             static_cast<const uint16_t*>(latent), ld_latent,
             cu_q, cu_k, q_row_ids, batch, n_qt, scale * kLog2e,
             out, out_row_stride, lse, lse_row_stride};
  dim3 g((unsigned)total);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const bool rid = q_row_ids != nullptr, c = causal != 0;
  if (NW == 8) launch1<8>(c, rid, out_dtype, g, s, a);
  else if (NW == 4) launch1<4>(c, rid, out_dtype, g, s, a);
  else launch1<2>(c, rid, out_dtype, g, s, a);
  return mla_check_launch("mla_prefill_attn");
}
