// Absorbed-form MLA attention (DeepSeek MLA -- Prefix Cache and Chunked
// Prefill, section 3: with W_UK folded into the query and W_UV applied after
// the attention, every head attends directly to the shared 576-wide latent,
// which serves as key [c_kv | k_rope] and, through its first 512 elements, as
// value). Used for query sets that are small next to the key count, where
// decompressing per-head K/V would cost more than it saves: the protected
// rows of the Local heads in head-partitioned reuse (RedKnot-MLA, section 2).
//
//   mla_absorb_q       q_abs = [q_nope W_UK^h^T | q_rope], one row per (head, row)
//   mla_absorbed_attn  multi-query flash attention of the q_abs rows over
//                      latent keys, per key piece: (o_lat [512], lse)
//   mla_absorb_out     out^h = o_lat W_UV^h
#include "mla_internal.h"

namespace {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazy = 8.f;   // log2 headroom of the lazy softmax reference

// ---------------------------------------------------------------- small batched GEMMs
//
// D[h][i][n] = sum_k A(h, i, k) Bt(h, n, k) for a few rows per head: one
// wavefront per 32 x 32 output tile, operands read straight from global
// memory (16 bytes per lane per k step), v_mfma_f32_32x32x16_bf16 issued as
// D^T = Bt_frag x A_frag so a lane holds four consecutive columns of one row.

struct AbsorbQArgs {
  const uint16_t* q; int64_t q_rs; int h_begin; const int32_t* row_ids; int n_rows;
  const uint16_t* kvb; int64_t ld_kvb;       // kv_b_proj [512][H_total * 256]
  uint16_t* qa;                              // [Hsel * n_rows][576]
};

struct AbsorbOutArgs {
  const uint16_t* ol; int n_rows;            // o_lat [Hsel * n_rows][512] bf16
  const uint16_t* wt; int H_total; int h_begin;   // packed weight [H_total * 256][512]
  uint16_t* out; int64_t out_rs;             // out [n_rows][Hsel * 128] (row stride out_rs)
};

__device__ __forceinline__ bf16x8 ld16(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

// tiles per head: ceil(n_rows / 32) row tiles x 18 column tiles (16 of the
// absorbed 512 columns, 2 of the copied rope part)
__global__ __launch_bounds__(256) void absorb_q_kernel(AbsorbQArgs a, int n_mt, int total) {
  const int lane = threadIdx.x & 63, l32 = lane & 31, g = lane >> 5;
  const int tile = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (tile >= total) return;
  const int per_head = n_mt * 18;
  const int hs = tile / per_head, rem = tile % per_head;
  const int mt = rem / 18, nt = rem % 18;
  const int i = mt * 32 + l32;                          // this lane's row
  const bool ok = i < a.n_rows;
  const int h = a.h_begin + hs;
  const uint16_t* qrow = a.q + (ok ? (int64_t)a.row_ids[i] : 0) * a.q_rs + (int64_t)h * kDqk;
  uint16_t* drow = a.qa + ((int64_t)hs * a.n_rows + i) * kDlat;
  if (nt >= 16) {
    // rope part: copy q[row][h][128 + 32 (nt - 16) + 16 g .. +16]
    if (ok) {
      const int c0 = 32 * (nt - 16) + 16 * g;
      *reinterpret_cast<u32x4*>(drow + kDc + c0) = *reinterpret_cast<const u32x4*>(qrow + kDnope + c0);
      *reinterpret_cast<u32x4*>(drow + kDc + c0 + 8) = *reinterpret_cast<const u32x4*>(qrow + kDnope + c0 + 8);
    }
    return;
  }
  // W_UK^h^T row j = kv_b_proj[j][h * 128 + (0..127)]
  const uint16_t* brow = a.kvb + (int64_t)(nt * 32 + l32) * a.ld_kvb + (int64_t)h * kDnope;
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  bf16x8 af[kDnope / 16], bf[kDnope / 16];
#pragma unroll
  for (int s = 0; s < kDnope / 16; ++s) {
    af[s] = ok ? ld16(qrow + 16 * s + 8 * g) : bf16x8{};
    bf[s] = ld16(brow + 16 * s + 8 * g);
  }
#pragma unroll
  for (int s = 0; s < kDnope / 16; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[s], af[s], acc, 0, 0, 0);
  if (!ok) return;
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) {
    const int n = nt * 32 + 8 * q4 + 4 * g;
    *reinterpret_cast<u32x2*>(drow + n) =
        u32x2{cvt_pk_bf16(acc[4 * q4], acc[4 * q4 + 1]), cvt_pk_bf16(acc[4 * q4 + 2], acc[4 * q4 + 3])};
  }
}

// tiles per head: ceil(n_rows / 32) x 4 (128 output columns)
__global__ __launch_bounds__(256) void absorb_out_kernel(AbsorbOutArgs a, int n_mt, int total) {
  const int lane = threadIdx.x & 63, l32 = lane & 31, g = lane >> 5;
  const int tile = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (tile >= total) return;
  const int per_head = n_mt * 4;
  const int hs = tile / per_head, rem = tile % per_head;
  const int mt = rem / 4, nt = rem % 4;
  const int i = mt * 32 + l32;
  const bool ok = i < a.n_rows;
  const uint16_t* arow = a.ol + ((int64_t)hs * a.n_rows + (ok ? i : 0)) * kDc;
  // W_UV^h^T row dv = packed weight row H_total * 128 + h * 128 + dv
  const uint16_t* brow = a.wt + ((int64_t)a.H_total * kDnope + (int64_t)(a.h_begin + hs) * kDv + nt * 32 + l32) * kDc;
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll 4
  for (int s = 0; s < kDc / 16; ++s) {
    const bf16x8 af = ok ? ld16(arow + 16 * s + 8 * g) : bf16x8{};
    const bf16x8 bf = ld16(brow + 16 * s + 8 * g);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf, af, acc, 0, 0, 0);
  }
  if (!ok) return;
  uint16_t* orow = a.out + (int64_t)i * a.out_rs + (int64_t)hs * kDv;
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) {
    const int n = nt * 32 + 8 * q4 + 4 * g;
    *reinterpret_cast<u32x2*>(orow + n) =
        u32x2{cvt_pk_bf16(acc[4 * q4], acc[4 * q4 + 1]), cvt_pk_bf16(acc[4 * q4 + 2], acc[4 * q4 + 3])};
  }
}

// ---------------------------------------------------------------- absorbed flash attention
//
// Workgroup = 128 query rows of one key piece, 4 wavefronts, one per SIMD;
// each wavefront owns 32 rows for all 576 query dims and all 512 value dims,
// so no partial sums cross wavefronts. Per 32-key tile:
//   scores    S^T[32 keys][32 rows] = K . Q^T over 36 k steps (Q in VGPRs,
//             two accumulator chains for the even and odd steps)
//   values    O^T[512 value dims][32 rows] += V^T P^T, 16 blocks of 32 x 32
//             (O, 256 registers, in the accumulation registers; one wavefront
//             per SIMD leaves them free)
// Every key and value fragment read from LDS feeds one product of 32 rows:
// 1 KB of LDS reads per 64 K flop, as in the decompressed-form attention.
// LDS per stage (36 KB): c_kv rows of 1024 B, 16-byte chunk c of key r at
// position c ^ f(r & 15), f(x) = ((x & 3) << 2) | (x >> 2), which keeps both
// the 16-byte key reads (16 keys, same chunk) and the transposing value reads
// free of bank conflicts; rope rows of 128 B, chunk c at c ^ ((r >> 1) & 7).
// Four stages; the DMA of tile t+3 is issued at step t (global_load_lds,
// keys past the piece end clamped to its last key and masked).
constexpr int kAT = 32;                         // keys per tile
constexpr int kACkv = kAT * 1024;               // c_kv region of a stage
constexpr int kAStage = kACkv + kAT * 128;      // + rope region = 36 KB
constexpr int kANB = 4;                         // stages
constexpr int kAW = 4;                          // wavefronts per workgroup
constexpr int kARows = 32 * kAW;                // query rows per workgroup
constexpr int kADma = 9;                        // DMA instructions per wavefront per tile

struct AbsAttnArgs {
  const uint16_t* qa; int R;                    // q_abs [R][576]
  const uint16_t* lat; int64_t ld;              // latent keys
  const int32_t* cu_k; int pieces; int n_rt; float scale_log2;
  void* out; float* lse4;                       // [pieces * R][512], [pieces * R][4]
};

__device__ __forceinline__ int akv_swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

template <int kOutDt>
__global__ __launch_bounds__(kAW * 64, 1) void absorbed_attn_kernel(AbsAttnArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kANB * kAStage];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;

  // Work items (piece, row tile), piece-major, are dealt to the 8 XCDs
  // (workgroup b runs on XCD b % 8) in contiguous ranges of equal size: the
  // row tiles of a piece share its keys in one XCD's L2 except where a range
  // boundary cuts the piece (a piece whose row tiles fit in a range lies on
  // at most two XCDs), and a launch of at most one workgroup per compute
  // unit runs in a single round whatever the piece count.
  const int n_items = a.pieces * a.n_rt;
  const int per_xcd = (n_items + 7) >> 3;
  const int slot = blockIdx.x >> 3;
  const int item = (blockIdx.x & 7) * per_xcd + slot;
  if (slot >= per_xcd || item >= n_items) return;
  const int pc = item / a.n_rt, rt = item % a.n_rt;
  const int k0 = a.cu_k[pc];
  const int n_k = a.cu_k[pc + 1] - k0;
  const int row = rt * kARows + wave * 32 + l32;
  const bool row_ok = row < a.R;
  const int ntiles = (n_k + kAT - 1) / kAT;

  // the 576 query dims of this lane's row as B fragments
  bf16x8 qf[kDlat / 16];
  {
    const uint16_t* qp = a.qa + (int64_t)(row_ok ? row : 0) * kDlat + 8 * g;
#pragma unroll
    for (int s = 0; s < kDlat / 16; ++s) qf[s] = row_ok ? ld16(qp + 16 * s) : bf16x8{};
  }

  // DMA: wavefront w moves c_kv rows w, w+4, ..., w+28 (1 KB each) and rope
  // rows 8w .. 8w+7; a lane's position is fixed, the global chunk it fetches
  // is the inverse swizzle (XOR is its own inverse)
  const int klast = n_k - 1;
  const uint16_t* base = a.lat + (int64_t)k0 * a.ld;
  // DMA of tile t into stage `stage`; the stage follows the step, not the
  // (clamped) tile index, so a clamped copy never lands in a stage still to
  // be read
  auto dma = [&](int t, int stage) __attribute__((always_inline)) {
    uint8_t* st = lds + stage * kAStage;
    const int kt0 = t * kAT;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = i * kAW + wave;
      const int c = lane ^ akv_swz(r & 15);
      const int key = min(kt0 + r, klast);
      dma16(base + (int64_t)key * a.ld + c * 8, st + r * 1024);
    }
    {
      const int r = 8 * wave + (lane >> 3);
      const int c = (lane & 7) ^ ((r >> 1) & 7);
      const int key = min(kt0 + r, klast);
      dma16(base + (int64_t)key * a.ld + kDc + c * 8, st + kACkv + wave * 1024);
    }
  };

  f32x16 O[16];
#pragma unroll
  for (int d = 0; d < 16; ++d)
#pragma unroll
    for (int i = 0; i < 16; ++i) O[d][i] = 0.f;
  float m_ref = -INFINITY, l_run = 0.f;
  const float c = a.scale_log2;

  // Fragment read offsets. Swizzles only touch the low four chunk bits, so
  // the offset of a read is one of a few per-lane bases plus a constant:
  //   key reads (key l32, query-dim step s, chunk 2 s + g): c_kv steps
  //   s < 32 use kb[s & 7] + 256 (s >> 3), rope steps kr[s - 32];
  //   value reads (transposing, 8 keys of one value column per lane over two
  //   reads; row 16 mm + 8 hi + 4 g + a4, value dims 32 d + 16 g16 + 4 b4)
  //   use vb[hi][d & 3] + 16384 mm + 256 (d >> 2).
  int kb[8], kr[4], vb[2][4];
  {
    const int sw = akv_swz(l32 & 15);
#pragma unroll
    for (int s8 = 0; s8 < 8; ++s8) kb[s8] = l32 * 1024 + (((2 * s8 + g) ^ sw) << 4);
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) kr[s4] = kACkv + l32 * 128 + (((2 * s4 + g) ^ ((l32 >> 1) & 7)) << 4);
    const int a4 = (lane & 15) >> 2, b4 = lane & 3, g16 = (lane >> 4) & 1;
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
      const int r = 8 * hi + 4 * g + a4;
#pragma unroll
      for (int d4 = 0; d4 < 4; ++d4)
        vb[hi][d4] = r * 1024 + (((4 * d4 + 2 * g16 + (b4 >> 1)) ^ akv_swz(r)) << 4) + 8 * (b4 & 1);
    }
  }
  auto koff = [&](int s) __attribute__((always_inline)) { return s < 32 ? kb[s & 7] + 256 * (s >> 3) : kr[s - 32]; };
  auto voff = [&](int mm, int hi, int d) __attribute__((always_inline)) {
    return vb[hi][d & 3] + 16384 * mm + 256 * (d >> 2);
  };

  // An empty piece issues no DMA at all: with no key there is no address to
  // clamp to, and the epilogue writes the identity state (0, -inf).
  if (ntiles > 0)
    for (int t = 0; t < kANB - 1; ++t) dma(min(t, ntiles - 1), t);
  wait_vmcnt<0>();
  for (int t = 0; t < ntiles; ++t) {
    // own DMA of tile t done (tiles t+1, t+2 may be in flight); then the
    // barrier publishes tile t and frees the stage of tile t-1
    wait_vmcnt<2 * kADma>();
    __syncthreads();
    dma(min(t + kANB - 1, ntiles - 1), (t + kANB - 1) % kANB);
    const uint8_t* st = lds + (t % kANB) * kAStage;
    const int kt0 = t * kAT;

    // scores: two chains (even and odd k steps), added at the end
    f32x16 S0, S1;
#pragma unroll
    for (int i = 0; i < 16; ++i) { S0[i] = 0.f; S1[i] = 0.f; }
#pragma unroll
    for (int s = 0; s < kDlat / 16; s += 2) {
      const bf16x8 k0f = *reinterpret_cast<const bf16x8*>(st + koff(s));
      const bf16x8 k1f = *reinterpret_cast<const bf16x8*>(st + koff(s + 1));
      S0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0f, qf[s], S0, 0, 0, 0);
      S1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1f, qf[s + 1], S1, 0, 0, 0);
    }
    // key fragment reads two ahead of the products
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
    for (int i = 0; i < 17; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    f32x16 S;
#pragma unroll
    for (int i = 0; i < 16; ++i) S[i] = S0[i] + S1[i];
    // keys past the piece end
    if (kt0 + kAT > n_k) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kt0 + 8 * (i >> 2) + 4 * g + (i & 3);
        S[i] = key < n_k ? S[i] : -INFINITY;
      }
    }
    // online softmax with a lazy reference max (log2 units), as in the
    // decompressed-form attention: row max over own 16 keys and lane l ^ 32
    float mt = S[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mt = fmaxf(mt, S[i]);
    {
      const uint32_t u = __float_as_uint(mt);
      const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
      mt = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    }
    const float mtc = mt * c;
    const bool bump = mtc > m_ref + kLazy;
    const float m_new = bump ? mtc : m_ref;
    const float alpha = bump ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.f;
    const float mc = (m_new == -INFINITY) ? 0.f : m_new;
    float ps = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = __builtin_amdgcn_exp2f(fmaf(S[i], c, -mc));
      S[i] = p;
      ps += p;
    }
    l_run = fmaf(l_run, alpha, ps);
    m_ref = m_new;
    if (__any(bump)) {
      // O stays in the accumulation registers: the factor is applied there
      // in place (plain code would keep a second copy of O alive)
#pragma unroll
      for (int d = 0; d < 16; ++d)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float tmp;
          asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                       : "+a"(O[d][i]), "=&v"(tmp)
                       : "v"(alpha));
        }
    }
    // O^T[value dims][rows] += V^T P^T over keys 16 mm .. 16 mm + 15
#pragma unroll
    for (int mm = 0; mm < 2; ++mm) {
      const int i0 = 8 * mm;
      const u32x4 u = {cvt_pk_bf16(S[i0], S[i0 + 1]), cvt_pk_bf16(S[i0 + 2], S[i0 + 3]),
                       cvt_pk_bf16(S[i0 + 4], S[i0 + 5]), cvt_pk_bf16(S[i0 + 6], S[i0 + 7])};
      const bf16x8 pf = __builtin_bit_cast(bf16x8, u);
#pragma unroll
      for (int d = 0; d < 16; ++d) {
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(st + voff(mm, 0, d)));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(st + voff(mm, 1, d)));
        const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        O[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, O[d], 0, 0, 0);
      }
    }
    // value fragment reads four ahead of the products
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 1);
#pragma unroll
    for (int i = 0; i < 30; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 1);
  }
  wait_vmcnt<0>();

  // ---- epilogue: row sums of the two lane halves; the 512 value dims and
  // four copies of the lse
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (!row_ok) return;
  const bool empty = !(l_tot > 0.f);
  const float inv = empty ? 0.f : 1.f / l_tot;
  const int64_t orow = (int64_t)pc * a.R + row;
#pragma unroll
  for (int d = 0; d < 16; ++d)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int dv = 32 * d + 8 * q4 + 4 * g;
      const float o0 = O[d][4 * q4] * inv, o1 = O[d][4 * q4 + 1] * inv;
      const float o2 = O[d][4 * q4 + 2] * inv, o3 = O[d][4 * q4 + 3] * inv;
      if (kOutDt == MLA_DTYPE_FP32) {
        *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + orow * kDc + dv) = f32x4{o0, o1, o2, o3};
      } else {
        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.out) + orow * kDc + dv) =
            u32x2{cvt_pk_bf16(o0, o1), cvt_pk_bf16(o2, o3)};
      }
    }
  if (g == 0) {
    const float lse = empty ? -INFINITY : (m_ref + __builtin_amdgcn_logf(l_tot)) * kLn2;
#pragma unroll
    for (int k = 0; k < 4; ++k) a.lse4[orow * 4 + k] = lse;
  }
}

}  // namespace

extern "C" int mla_absorb_q(const void* q, int64_t q_row_stride, int H_q, int h_begin, int h_end,
                            const int32_t* row_ids, int n_rows, const void* kv_b_proj, int H_total,
                            void* q_abs, void* stream) {
  mla_begin_call();
  MLA_REQUIRE(n_rows >= 0, MLA_ERR_INVALID_ARG, "mla_absorb_q: n_rows must be >= 0");
  MLA_REQUIRE(H_q > 0 && 0 <= h_begin && h_begin < h_end && h_end <= H_q && h_end <= H_total, MLA_ERR_INVALID_ARG,
              "mla_absorb_q: need 0 <= h_begin (%d) < h_end (%d) <= min(H_q (%d), H_total (%d))", h_begin, h_end,
              H_q, H_total);
  if (n_rows == 0) return MLA_OK;
  MLA_REQUIRE(q && row_ids && kv_b_proj && q_abs, MLA_ERR_INVALID_ARG, "mla_absorb_q: null pointer argument");
  MLA_REQUIRE(mla_aligned16(q) && mla_aligned16(kv_b_proj) && mla_aligned16(q_abs), MLA_ERR_INVALID_ARG,
              "mla_absorb_q: pointers must be 16-byte aligned");
  MLA_REQUIRE(q_row_stride % 8 == 0 && q_row_stride >= (int64_t)H_q * kDqk, MLA_ERR_INVALID_ARG,
              "mla_absorb_q: q_row_stride must be a multiple of 8 and >= H_q*192");
  const int Hsel = h_end - h_begin;
  const int n_mt = (n_rows + 31) / 32;
  const int64_t total = (int64_t)Hsel * n_mt * 18;
  MLA_REQUIRE(total < (int64_t)1 << 30, MLA_ERR_INVALID_ARG, "mla_absorb_q: problem too large");
  AbsorbQArgs a{static_cast<const uint16_t*>(q), q_row_stride, h_begin, row_ids, n_rows,
                static_cast<const uint16_t*>(kv_b_proj), (int64_t)H_total * 2 * kDnope,
                static_cast<uint16_t*>(q_abs)};
  hipLaunchKernelGGL(absorb_q_kernel, dim3((unsigned)((total + 3) / 4)), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), a, n_mt, (int)total);
  return mla_check_launch("mla_absorb_q");
}

extern "C" int mla_absorbed_attn(const void* q_abs, int R, const void* latent, int64_t ld_latent,
                                 const int32_t* cu_k, int pieces, float scale, void* out_lat, int out_dtype,
                                 float* lse4, void* stream) {
  mla_begin_call();
  MLA_REQUIRE(R >= 0 && pieces >= 0, MLA_ERR_INVALID_ARG, "mla_absorbed_attn: R and pieces must be >= 0");
  if (R == 0 || pieces == 0) return MLA_OK;
  MLA_REQUIRE(q_abs && latent && cu_k && out_lat && lse4, MLA_ERR_INVALID_ARG,
              "mla_absorbed_attn: null pointer argument");
  MLA_REQUIRE(out_dtype == MLA_DTYPE_BF16 || out_dtype == MLA_DTYPE_FP32, MLA_ERR_UNSUPPORTED,
              "mla_absorbed_attn: out dtype %d not supported", out_dtype);
  MLA_REQUIRE(mla_aligned16(q_abs) && mla_aligned16(latent) && mla_aligned16(out_lat), MLA_ERR_INVALID_ARG,
              "mla_absorbed_attn: pointers must be 16-byte aligned");
  MLA_REQUIRE(ld_latent % 8 == 0 && ld_latent >= kDlat, MLA_ERR_INVALID_ARG,
              "mla_absorbed_attn: ld_latent (%lld) must be a multiple of 8 and >= 576", (long long)ld_latent);
  MLA_REQUIRE(scale > 0.f && scale < 1e30f, MLA_ERR_INVALID_ARG, "mla_absorbed_attn: scale must be positive");
  const int n_rt = (R + kARows - 1) / kARows;
  const int64_t total = ((int64_t)pieces * n_rt + 7) / 8 * 8;   // 8 equal per-XCD ranges of work items
  MLA_REQUIRE(total < (int64_t)1 << 31, MLA_ERR_INVALID_ARG, "mla_absorbed_attn: problem too large");
  AbsAttnArgs a{static_cast<const uint16_t*>(q_abs), R, static_cast<const uint16_t*>(latent), ld_latent,
                cu_k, pieces, n_rt, scale * kLog2e, out_lat, lse4};
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (out_dtype == MLA_DTYPE_FP32)
    hipLaunchKernelGGL(absorbed_attn_kernel<MLA_DTYPE_FP32>, dim3((unsigned)total), dim3(kAW * 64), 0, s, a);
  else
    hipLaunchKernelGGL(absorbed_attn_kernel<MLA_DTYPE_BF16>, dim3((unsigned)total), dim3(kAW * 64), 0, s, a);
  return mla_check_launch("mla_absorbed_attn");
}

extern "C" int mla_absorb_out(const void* o_lat, int n_rows, const void* w_t, int H_total, int h_begin, int h_end,
                              void* out, int64_t out_row_stride, void* stream) {
  mla_begin_call();
  MLA_REQUIRE(n_rows >= 0, MLA_ERR_INVALID_ARG, "mla_absorb_out: n_rows must be >= 0");
  MLA_REQUIRE(H_total > 0 && 0 <= h_begin && h_begin < h_end && h_end <= H_total, MLA_ERR_INVALID_ARG,
              "mla_absorb_out: need 0 <= h_begin (%d) < h_end (%d) <= H_total (%d)", h_begin, h_end, H_total);
  if (n_rows == 0) return MLA_OK;
  MLA_REQUIRE(o_lat && w_t && out, MLA_ERR_INVALID_ARG, "mla_absorb_out: null pointer argument");
  MLA_REQUIRE(mla_aligned16(o_lat) && mla_aligned16(w_t) && mla_aligned16(out), MLA_ERR_INVALID_ARG,
              "mla_absorb_out: pointers must be 16-byte aligned");
  const int Hsel = h_end - h_begin;
  MLA_REQUIRE(out_row_stride % 4 == 0 && out_row_stride >= (int64_t)Hsel * kDv, MLA_ERR_INVALID_ARG,
              "mla_absorb_out: out_row_stride must be a multiple of 4 and >= (h_end-h_begin)*128");
  const int n_mt = (n_rows + 31) / 32;
  const int64_t total = (int64_t)Hsel * n_mt * 4;
  MLA_REQUIRE(total < (int64_t)1 << 30, MLA_ERR_INVALID_ARG, "mla_absorb_out: problem too large");
  AbsorbOutArgs a{static_cast<const uint16_t*>(o_lat), n_rows, static_cast<const uint16_t*>(w_t), H_total, h_begin,
                  static_cast<uint16_t*>(out), out_row_stride};
  hipLaunchKernelGGL(absorb_out_kernel, dim3((unsigned)((total + 3) / 4)), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), a, n_mt, (int)total);
  return mla_check_launch("mla_absorb_out");
}
