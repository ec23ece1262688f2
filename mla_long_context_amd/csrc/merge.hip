// Log-sum-exp merge of two attention states (DeepSeek MLA -- Prefix Cache and
// Chunked Prefill, section 4.3 merge_attn_states; the merged lse that the
// chunk loop of section 4.4 consumes is m + ln(wa + wb)).
//
// HBM-bound. 16 lanes own one 128-wide state row, 8 values per lane, so a
// wavefront streams 4 rows of each operand with 16- or 32-byte accesses.
#include "mla_internal.h"

namespace {

constexpr int kThreads = 256;

template <int kDt>
struct Vec8;
template <>
struct Vec8<MLA_DTYPE_BF16> {
  __device__ static void load(const void* p, int64_t off, float* f) {
    const u32x4 u = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(p) + off);
    f[0] = bf16_bits_to_f32(u.x & 0xffffu); f[1] = bf16_bits_to_f32(u.x >> 16);
    f[2] = bf16_bits_to_f32(u.y & 0xffffu); f[3] = bf16_bits_to_f32(u.y >> 16);
    f[4] = bf16_bits_to_f32(u.z & 0xffffu); f[5] = bf16_bits_to_f32(u.z >> 16);
    f[6] = bf16_bits_to_f32(u.w & 0xffffu); f[7] = bf16_bits_to_f32(u.w >> 16);
  }
  __device__ static void store(void* p, int64_t off, const float* f) {
    u32x4 u;
    u.x = pack_bf16x2(f[0], f[1]); u.y = pack_bf16x2(f[2], f[3]);
    u.z = pack_bf16x2(f[4], f[5]); u.w = pack_bf16x2(f[6], f[7]);
    *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(p) + off) = u;
  }
};
template <>
struct Vec8<MLA_DTYPE_FP32> {
  __device__ static void load(const void* p, int64_t off, float* f) {
    const f32x4* q = reinterpret_cast<const f32x4*>(static_cast<const float*>(p) + off);
    const f32x4 a = q[0], b = q[1];
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
    f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  }
  __device__ static void store(void* p, int64_t off, const float* f) {
    f32x4* q = reinterpret_cast<f32x4*>(static_cast<float*>(p) + off);
    q[0] = f32x4{f[0], f[1], f[2], f[3]};
    q[1] = f32x4{f[4], f[5], f[6], f[7]};
  }
};

template <int kDa, int kDb, int kDo>
__global__ __launch_bounds__(kThreads) void merge_kernel(const void* oa, const float* la,
                                                          const void* ob, const float* lb,
                                                          int64_t rows, void* out, float* lo) {
  const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t row = gid >> 4;
  const int part = (int)(gid & 15);
  if (row >= rows) return;
  const float a = la[row], b = lb[row];
  const float m = fmaxf(a, b);
  const int64_t off = row * kDv + part * 8;
  float r[8];
  float lse;
  if (m == -INFINITY) {
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = 0.f;
    lse = -INFINITY;
  } else {
    const float wa = (a == -INFINITY) ? 0.f : expf(a - m);
    const float wb = (b == -INFINITY) ? 0.f : expf(b - m);
    const float s = wa + wb;
    const float ca = wa / s, cb = wb / s;
    float fa[8], fb[8];
    if (wa != 0.f) Vec8<kDa>::load(oa, off, fa);
    else {
#pragma unroll
      for (int j = 0; j < 8; ++j) fa[j] = 0.f;
    }
    if (wb != 0.f) Vec8<kDb>::load(ob, off, fb);
    else {
#pragma unroll
      for (int j = 0; j < 8; ++j) fb[j] = 0.f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = ca * fa[j] + cb * fb[j];
    lse = m + logf(s);
  }
  Vec8<kDo>::store(out, off, r);
  if (part == 0) lo[row] = lse;
}

template <int kDa, int kDb>
int launch_o(int dto, dim3 g, hipStream_t s, const void* oa, const float* la, const void* ob,
             const float* lb, int64_t rows, void* out, float* lo) {
  if (dto == MLA_DTYPE_BF16)
    hipLaunchKernelGGL((merge_kernel<kDa, kDb, MLA_DTYPE_BF16>), g, dim3(kThreads), 0, s, oa, la, ob, lb, rows, out, lo);
  else
    hipLaunchKernelGGL((merge_kernel<kDa, kDb, MLA_DTYPE_FP32>), g, dim3(kThreads), 0, s, oa, la, ob, lb, rows, out, lo);
  return mla_check_launch("mla_merge_states");
}

template <int kDa>
int launch_b(int dtb, int dto, dim3 g, hipStream_t s, const void* oa, const float* la,
             const void* ob, const float* lb, int64_t rows, void* out, float* lo) {
  if (dtb == MLA_DTYPE_BF16) return launch_o<kDa, MLA_DTYPE_BF16>(dto, g, s, oa, la, ob, lb, rows, out, lo);
  return launch_o<kDa, MLA_DTYPE_FP32>(dto, g, s, oa, la, ob, lb, rows, out, lo);
}

// The merge of `pieces` states per row in one pass (the merge of the same
// section applied to all of them at once, which by its identity equals any
// order of pairwise merges): m = max_p l_p, w_p = e^{l_p - m} (0 for a piece
// at -inf), out = sum_p w_p o_p / sum_p w_p, lse = m + ln sum_p w_p.
//
// A workgroup owns 4 rows (16 lanes per row, 8 values per lane) and W <= 8
// wavefronts; wavefront w folds pieces w, w + W, w + 2W, ... into a running
// state (m, s, r) with the usual rescaling by e^{m_old - m_new}, four pieces'
// loads in flight per round. Wavefront 0 then folds the W states from LDS in
// wavefront order, so the result does not depend on timing. Splitting the
// pieces over wavefronts keeps many loads in flight when there are few rows
// and many pieces (thousands of rows, tens of pieces). Every state is read
// once, before anything is written, so the output may alias piece 0.
constexpr int kMaxW = 8;    // wavefronts per workgroup, at most
constexpr int kPer = 4;     // pieces whose loads one wavefront issues together

// Several independent merges in one launch (the sets of
// mla_merge_states_sets): set k owns workgroups [first[k], first[k+1]).
// A wavefront of a set with fewer pieces than wavefronts folds nothing and
// hands the empty state (-inf, 0, 0) to the combine.
struct MergeSetDev {
  const void* outs; const float* lses; int pieces; int64_t rows; void* out; float* lo;
};
struct MergeSetsDev {
  MergeSetDev s[MLA_MERGE_MAX_SETS];
  int64_t first[MLA_MERGE_MAX_SETS + 1];
  int n;
};

template <int kDi, int kDo>
__global__ __launch_bounds__(kMaxW * 64) void merge_n_kernel(MergeSetsDev ms) {
  __shared__ float sh[kMaxW - 1][10][64];      // [wavefront 1..W-1][m, s, r0..r7][lane]
  // this workgroup's set (wavefront-uniform, a few scalar compares)
  int64_t blk = blockIdx.x;
  int k = 0;
#pragma unroll
  for (int j = 1; j < MLA_MERGE_MAX_SETS; ++j)
    if (j < ms.n && blk >= ms.first[j]) k = j;
  blk -= ms.first[k];
  const void* outs = ms.s[0].outs; const float* lses = ms.s[0].lses; int pieces = ms.s[0].pieces;
  int64_t rows = ms.s[0].rows; void* out = ms.s[0].out; float* lo = ms.s[0].lo;
#pragma unroll
  for (int j = 1; j < MLA_MERGE_MAX_SETS; ++j)
    if (k == j) {
      outs = ms.s[j].outs; lses = ms.s[j].lses; pieces = ms.s[j].pieces;
      rows = ms.s[j].rows; out = ms.s[j].out; lo = ms.s[j].lo;
    }
  const int W = (int)(blockDim.x >> 6);
  const int wave = (int)(threadIdx.x >> 6), lane = (int)(threadIdx.x & 63);
  const int64_t row = blk * 4 + (lane >> 4);
  const bool live = row < rows;
  const int64_t off = row * kDv + (lane & 15) * 8;
  float m = -INFINITY, s = 0.f, r[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = 0.f;
  if (live) {
    for (int p0 = wave; p0 < pieces; p0 += kPer * W) {
      float l[kPer], f[kPer][8];
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        const int p = p0 + k * W;
        l[k] = -INFINITY;
#pragma unroll
        for (int j = 0; j < 8; ++j) f[k][j] = 0.f;
        if (p < pieces) {
          l[k] = lses[(int64_t)p * rows + row];
          Vec8<kDi>::load(outs, (int64_t)p * rows * kDv + off, f[k]);
        }
      }
      float mn = m;
#pragma unroll
      for (int k = 0; k < kPer; ++k) mn = fmaxf(mn, l[k]);
      if (mn == -INFINITY) continue;
      const float c = expf(m - mn);              // 0 while the state is empty
      s *= c;
#pragma unroll
      for (int j = 0; j < 8; ++j) r[j] *= c;
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        const float w = (l[k] == -INFINITY) ? 0.f : expf(l[k] - mn);
        s += w;
        // a piece of weight 0 contributes nothing, whatever its values hold
#pragma unroll
        for (int j = 0; j < 8; ++j) r[j] = fmaf(w, w != 0.f ? f[k][j] : 0.f, r[j]);
      }
      m = mn;
    }
  }
  if (W > 1) {
    if (wave > 0) {
      sh[wave - 1][0][lane] = m;
      sh[wave - 1][1][lane] = s;
#pragma unroll
      for (int j = 0; j < 8; ++j) sh[wave - 1][2 + j][lane] = r[j];
    }
    __syncthreads();
    if (wave > 0) return;
    for (int v = 0; v < W - 1; ++v) {
      const float m2 = sh[v][0][lane];
      const float mn = fmaxf(m, m2);
      if (mn == -INFINITY) continue;
      const float ca = expf(m - mn), cb = expf(m2 - mn);
      s = s * ca + sh[v][1][lane] * cb;
#pragma unroll
      for (int j = 0; j < 8; ++j) r[j] = r[j] * ca + sh[v][2 + j][lane] * cb;
      m = mn;
    }
  }
  if (!live) return;
  float lse = -INFINITY;
  if (m != -INFINITY) {
    const float inv = 1.f / s;
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] *= inv;
    lse = m + logf(s);
  }
  Vec8<kDo>::store(out, off, r);
  if ((lane & 15) == 0) lo[row] = lse;
}

bool ok_dt(int d) { return d == MLA_DTYPE_BF16 || d == MLA_DTYPE_FP32; }

}  // namespace

extern "C" int mla_merge_states(const void* out_a, int dtype_a, const float* lse_a,
                                const void* out_b, int dtype_b, const float* lse_b,
                                int64_t rows, void* out, int dtype_out, float* lse_out,
                                void* stream) {
  mla_begin_call();
  MLA_REQUIRE(rows >= 0, MLA_ERR_INVALID_ARG, "mla_merge_states: rows (%lld) must be >= 0", (long long)rows);
  if (rows == 0) return MLA_OK;
  MLA_REQUIRE(out_a && lse_a && out_b && lse_b && out && lse_out, MLA_ERR_INVALID_ARG,
              "mla_merge_states: null pointer argument");
  MLA_REQUIRE(ok_dt(dtype_a) && ok_dt(dtype_b) && ok_dt(dtype_out), MLA_ERR_UNSUPPORTED,
              "mla_merge_states: dtypes must be bf16 or fp32 (got %d, %d, %d)", dtype_a, dtype_b, dtype_out);
  MLA_REQUIRE(mla_aligned16(out_a) && mla_aligned16(out_b) && mla_aligned16(out), MLA_ERR_INVALID_ARG,
              "mla_merge_states: state pointers must be 16-byte aligned");
  // 16 lanes per row: the grid has rows / 16 workgroups, at most 2^31 - 1
  MLA_REQUIRE(rows <= (int64_t)1 << 34, MLA_ERR_INVALID_ARG, "mla_merge_states: rows (%lld) too large for one call",
              (long long)rows);
  const int64_t threads = rows * 16;
  dim3 g((unsigned)((threads + kThreads - 1) / kThreads));
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (dtype_a == MLA_DTYPE_BF16)
    return launch_b<MLA_DTYPE_BF16>(dtype_b, dtype_out, g, s, out_a, lse_a, out_b, lse_b, rows, out, lse_out);
  return launch_b<MLA_DTYPE_FP32>(dtype_b, dtype_out, g, s, out_a, lse_a, out_b, lse_b, rows, out, lse_out);
}

namespace {

// validation and launch shared by mla_merge_states_n and mla_merge_states_sets
int merge_sets(const char* fn, const MlaMergeSet* sets, int n_sets, int dtype_in, int dtype_out, void* stream) {
  MLA_REQUIRE(ok_dt(dtype_in) && ok_dt(dtype_out), MLA_ERR_UNSUPPORTED,
              "%s: dtypes must be bf16 or fp32 (got %d, %d)", fn, dtype_in, dtype_out);
  MergeSetsDev ms{};
  int64_t total = 0;
  int W = 1;
  for (int k = 0; k < n_sets; ++k) {
    const MlaMergeSet& t = sets[k];
    MLA_REQUIRE(t.rows >= 0 && t.pieces >= 1, MLA_ERR_INVALID_ARG,
                "%s: set %d needs rows (%lld) >= 0 and pieces (%d) >= 1", fn, k, (long long)t.rows, t.pieces);
    if (t.rows > 0) {
      MLA_REQUIRE(t.outs && t.lses && t.out && t.lse_out, MLA_ERR_INVALID_ARG, "%s: set %d: null pointer", fn, k);
      MLA_REQUIRE(mla_aligned16(t.outs) && mla_aligned16(t.out), MLA_ERR_INVALID_ARG,
                  "%s: set %d: state pointers must be 16-byte aligned", fn, k);
      MLA_REQUIRE(t.rows <= (int64_t)1 << 40 && (int64_t)t.pieces * t.rows <= (int64_t)1 << 40,
                  MLA_ERR_INVALID_ARG, "%s: set %d: rows too large", fn, k);
      // as many wavefronts per 4-row group as the set with most pieces has, up to 8
      const int wk = t.pieces < kMaxW ? t.pieces : kMaxW;
      if (wk > W) W = wk;
    }
    ms.s[k] = MergeSetDev{t.outs, t.lses, t.pieces, t.rows, t.out, t.lse_out};
    ms.first[k] = total;
    total += (t.rows + 3) / 4;
  }
  ms.first[n_sets] = total;
  ms.n = n_sets;
  if (total == 0) return MLA_OK;
  MLA_REQUIRE(total <= 0x7fffffff, MLA_ERR_INVALID_ARG, "%s: rows too large for one call", fn);
  dim3 g((unsigned)total), blk((unsigned)(W * 64));
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (dtype_in == MLA_DTYPE_BF16) {
    if (dtype_out == MLA_DTYPE_BF16)
      hipLaunchKernelGGL((merge_n_kernel<MLA_DTYPE_BF16, MLA_DTYPE_BF16>), g, blk, 0, s, ms);
    else
      hipLaunchKernelGGL((merge_n_kernel<MLA_DTYPE_BF16, MLA_DTYPE_FP32>), g, blk, 0, s, ms);
  } else {
    if (dtype_out == MLA_DTYPE_BF16)
      hipLaunchKernelGGL((merge_n_kernel<MLA_DTYPE_FP32, MLA_DTYPE_BF16>), g, blk, 0, s, ms);
    else
      hipLaunchKernelGGL((merge_n_kernel<MLA_DTYPE_FP32, MLA_DTYPE_FP32>), g, blk, 0, s, ms);
  }
  return mla_check_launch(fn);
}

}  // namespace

extern "C" int mla_merge_states_n(const void* outs, int dtype_in, const float* lses, int pieces, int64_t rows,
                                  void* out, int dtype_out, float* lse_out, void* stream) {
  mla_begin_call();
  MLA_REQUIRE(rows >= 0 && pieces >= 1, MLA_ERR_INVALID_ARG,
              "mla_merge_states_n: need rows (%lld) >= 0 and pieces (%d) >= 1", (long long)rows, pieces);
  if (rows == 0) return MLA_OK;
  const MlaMergeSet set{outs, lses, pieces, rows, out, lse_out};
  return merge_sets("mla_merge_states_n", &set, 1, dtype_in, dtype_out, stream);
}

extern "C" int mla_merge_states_sets(const MlaMergeSet* sets, int n_sets, int dtype_in, int dtype_out,
                                     void* stream) {
  mla_begin_call();
  MLA_REQUIRE(n_sets >= 0 && n_sets <= MLA_MERGE_MAX_SETS, MLA_ERR_INVALID_ARG,
              "mla_merge_states_sets: n_sets (%d) must be in [0, %d]", n_sets, MLA_MERGE_MAX_SETS);
  if (n_sets == 0) return MLA_OK;
  MLA_REQUIRE(sets, MLA_ERR_INVALID_ARG, "mla_merge_states_sets: null sets");
  return merge_sets("mla_merge_states_sets", sets, n_sets, dtype_in, dtype_out, stream);
}
