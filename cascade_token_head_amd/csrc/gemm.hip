// Q/K/V and output projections of the kept heads (SpAtten, section II
// "Attention mechanism": inputs split into per-head Q, K, V; head outputs
// concatenated; "Cascade pruning": a pruned head's Q/K/V chunks are gone).
//
// bf16 path: 128x128x64 workgroup tiles on gfx950 MFMA 32x32x16 (fp32
// accumulate), four waves of 64x64, operands staged through padded LDS
// rows with double buffering. Head pruning is a gather: each output
// column block (QKV) or K block (output projection) reads the weight rows
// or columns of the head kept in that slot, per sequence. When every head
// is kept all sequences share the weights and M tiles run across sequence
// boundaries; otherwise M tiles stay inside one sequence.
// fp32 path: a plain 64x64 VALU tile for the fp32 workload.
#include "common.hpp"
#include "kernels.hpp"
#include "timing.hpp"

namespace spatten {
namespace {

enum { kQkvPrefill = 0, kQkvDecode = 1, kOut = 2 };

struct GemmParams {
  const void* A;
  int64_t lda;
  const void* W0;
  const void* W1;
  const void* W2;
  int64_t ldw;
  const int32_t* head_idx;
  int batch, n, seq_tiled, mt_per_seq, M_total, N, K;
  int h_kept, dh, D, n_pad;
  void* out0;
  void* out1;
  void* out2;
  int64_t kv_bs;
};

// Row of M tile `mt_flat`, local row r -> (valid, sequence, row in sequence)
struct RowMap {
  bool valid;
  int b, m;
};

__device__ __forceinline__ RowMap map_row(const GemmParams& p, int tile_y, int r, int BM) {
  RowMap rm;
  if (p.seq_tiled) {
    rm.b = tile_y / p.mt_per_seq;
    rm.m = (tile_y - rm.b * p.mt_per_seq) * BM + r;
    rm.valid = rm.m < p.n;
  } else {
    const int g = tile_y * BM + r;
    rm.valid = g < p.M_total;
    rm.b = g / p.n;
    rm.m = g - rm.b * p.n;
  }
  return rm;
}

__device__ __forceinline__ int head_of(const GemmParams& p, int b, int s) {
  return p.seq_tiled ? p.head_idx[b * p.h_kept + s] : s;
}

// Weight row (QKV) for output column ncol of sequence b.
template <typename T>
__device__ __forceinline__ const T* qkv_weight_row(const GemmParams& p, int b, int ncol) {
  const int hd = p.h_kept * p.dh;
  const int which = ncol / hd;
  const int rem = ncol - which * hd;
  const int s = rem / p.dh, c = rem - s * p.dh;
  const void* W = which == 0 ? p.W0 : (which == 1 ? p.W1 : p.W2);
  return static_cast<const T*>(W) + int64_t(head_of(p, b, s) * p.dh + c) * p.ldw;
}

template <typename T, int MODE>
__device__ __forceinline__ void store_out(const GemmParams& p, const RowMap& rm, int ncol,
                                          float v) {
  if (MODE == kOut) {
    const int64_t i = (int64_t(rm.b) * p.n + rm.m) * p.D + ncol;
    store_elem<T>(p.out0, i, load_elem<T>(p.out0, i) + v);
    return;
  }
  const int hd = p.h_kept * p.dh;
  const int which = ncol / hd;
  const int rem = ncol - which * hd;
  const int s = rem / p.dh, c = rem - s * p.dh;
  if (MODE == kQkvDecode) {
    if (which == 0)
      store_elem<T>(p.out0, int64_t(rm.b) * p.D + rem, v);
    else
      store_elem<T>(which == 1 ? p.out1 : p.out2, int64_t(rm.b) * p.kv_bs + rem, v);
    return;
  }
  const int64_t bs = int64_t(rm.b) * p.h_kept + s;
  if (which < 2)
    store_elem<T>(which == 0 ? p.out0 : p.out1, (bs * p.n_pad + rm.m) * p.dh + c, v);
  else
    store_elem<T>(p.out2, (bs * p.dh + c) * p.n_pad + rm.m, v);
}

// ------------------------------------------------------------------ bf16 MFMA

constexpr int BM = 128, BN = 128, BK = 64, LDS_K = BK + 8;

template <int MODE>
__global__ void __launch_bounds__(256)
gemm_bf16_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(16))) bf16_t As[2][BM * LDS_K];
  __shared__ __attribute__((aligned(16))) bf16_t Bs[2][BN * LDS_K];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tile_y = blockIdx.y, n0 = blockIdx.x * BN;
  const int b_tile = p.seq_tiled ? tile_y / p.mt_per_seq : 0;

  // global -> LDS assignment: 4 chunks of 16 B per thread for each operand
  const bf16_t* a_src[4];
  const bf16_t* w_src[4];
  int ld_row[4];
  const int kc = (tid & 7) * 8;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (tid >> 3) + 32 * i;
    ld_row[i] = r;
    RowMap rm = map_row(p, tile_y, r, BM);
    if (!rm.valid) {  // clamp to a real row; its results are never stored
      rm = p.seq_tiled ? RowMap{true, rm.b, p.n - 1} : RowMap{true, p.batch - 1, p.n - 1};
    }
    a_src[i] = static_cast<const bf16_t*>(p.A) + (int64_t(rm.b) * p.n + rm.m) * p.lda + kc;
    int ncol = n0 + r;
    if (ncol >= p.N) ncol = p.N - 1;
    if (MODE == kOut)
      w_src[i] = static_cast<const bf16_t*>(p.W0) + int64_t(ncol) * p.ldw;
    else
      w_src[i] = qkv_weight_row<bf16_t>(p, b_tile, ncol) + kc;
  }

  const int KT = p.K / BK;
  u32x4 ra[4], rb[4];
  auto gload = [&](int kt) {
    const int k0 = kt * BK;
    int wcol = k0;
    if (MODE == kOut) {
      const int s = k0 / p.dh;
      wcol = head_of(p, b_tile, s) * p.dh + (k0 - s * p.dh) + kc;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ra[i] = *reinterpret_cast<const u32x4*>(a_src[i] + k0);
      rb[i] = *reinterpret_cast<const u32x4*>(MODE == kOut ? w_src[i] + wcol : w_src[i] + k0);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<u32x4*>(&As[buf][ld_row[i] * LDS_K + kc]) = ra[i];
      *reinterpret_cast<u32x4*>(&Bs[buf][ld_row[i] * LDS_K + kc]) = rb[i];
    }
  };

  floatx16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
  const int fr = lane & 31, fk = (lane >> 5) * 8;

  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) gload(kt + 1);
#pragma unroll
    for (int kk = 0; kk < BK; kk += 16) {
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = as_bf16x8(*reinterpret_cast<const u32x4*>(
            &As[buf][(wm + 32 * i + fr) * LDS_K + kk + fk]));
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bfr[j] = as_bf16x8(*reinterpret_cast<const u32x4*>(
            &Bs[buf][(wn + 32 * j + fr) * LDS_K + kk + fk]));
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32x32x16(af[i], bfr[j], acc[i][j]);
    }
    if (kt + 1 < KT) sstore(buf ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int lr = wm + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      const RowMap rm = map_row(p, tile_y, lr, BM);
      if (!rm.valid) continue;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int ncol = n0 + wn + 32 * j + fr;
        if (ncol < p.N) store_out<bf16_t, MODE>(p, rm, ncol, acc[i][j][r]);
      }
    }
  }
}

// ------------------------------------------------------------------ fp32 VALU

constexpr int FT = 64, FK = 16;

template <int MODE>
__global__ void __launch_bounds__(256)
gemm_f32_kernel(GemmParams p) {
  __shared__ float As[FK][FT + 4];
  __shared__ float Bs[FK][FT + 4];
  const int tid = threadIdx.x;
  const int tile_y = blockIdx.y, n0 = blockIdx.x * FT;
  const int b_tile = p.seq_tiled ? tile_y / p.mt_per_seq : 0;
  const int tr = (tid >> 4) * 4, tc = (tid & 15) * 4;
  float acc[4][4] = {};
  // loader: 64 rows x 16 k per operand, 4 elements per thread
  const int lr = tid >> 2, lk = (tid & 3) * 4;
  RowMap rm = map_row(p, tile_y, lr, FT);
  if (!rm.valid) rm = p.seq_tiled ? RowMap{true, rm.b, p.n - 1} : RowMap{true, p.batch - 1, p.n - 1};
  const float* a_row = static_cast<const float*>(p.A) + (int64_t(rm.b) * p.n + rm.m) * p.lda;
  int ncol = n0 + lr;
  if (ncol >= p.N) ncol = p.N - 1;
  const float* w_row = MODE == kOut ? static_cast<const float*>(p.W0) + int64_t(ncol) * p.ldw
                                    : qkv_weight_row<float>(p, b_tile, ncol);
  for (int k0 = 0; k0 < p.K; k0 += FK) {
    int wcol = k0;
    if (MODE == kOut) {
      const int s = k0 / p.dh;
      wcol = head_of(p, b_tile, s) * p.dh + (k0 - s * p.dh);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      As[lk + e][lr] = a_row[k0 + lk + e];
      Bs[lk + e][lr] = w_row[wcol + lk + e];
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < FK; ++kk) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = As[kk][tr + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) bv[j] = Bs[kk][tc + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const RowMap om = map_row(p, tile_y, tr + i, FT);
    if (!om.valid) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = n0 + tc + j;
      if (c < p.N) store_out<float, MODE>(p, om, c, acc[i][j]);
    }
  }
}

template <int MODE>
int run_gemm(GemmParams& p, int dtype, hipStream_t stream) {
  const char* name = MODE == kOut ? "out_gemm" : "qkv_gemm";
  const int tm = dtype == SPATTEN_BF16 ? BM : FT;
  const int tn = dtype == SPATTEN_BF16 ? BN : FT;
  int tiles_y;
  if (p.seq_tiled) {
    p.mt_per_seq = int(ceil_div(p.n, tm));
    tiles_y = p.mt_per_seq * p.batch;
  } else {
    p.mt_per_seq = 0;
    tiles_y = int(ceil_div(p.M_total, tm));
  }
  const dim3 grid(unsigned(ceil_div(p.N, tn)), unsigned(tiles_y));
  if (dtype == SPATTEN_BF16)
    SPATTEN_TIMED(name, stream, gemm_bf16_kernel<MODE><<<grid, 256, 0, stream>>>(p));
  else
    SPATTEN_TIMED(name, stream, gemm_f32_kernel<MODE><<<grid, 256, 0, stream>>>(p));
  SPATTEN_LAUNCH_CHECK();
  return SPATTEN_OK;
}

}  // namespace

int launch_qkv(const QkvArgs& a, hipStream_t stream) {
  GemmParams p{};
  p.A = a.x;
  p.lda = a.D;
  p.W0 = a.w[0];
  p.W1 = a.w[1];
  p.W2 = a.w[2];
  p.ldw = a.D;
  p.head_idx = a.head_idx;
  p.batch = a.batch;
  p.n = a.n;
  p.seq_tiled = a.h_kept != a.D / a.dh;
  p.M_total = a.batch * a.n;
  p.N = 3 * a.h_kept * a.dh;
  p.K = a.D;
  p.h_kept = a.h_kept;
  p.dh = a.dh;
  p.D = a.D;
  p.n_pad = a.n_pad;
  p.out0 = a.q;
  p.out1 = a.k;
  p.out2 = a.vt;
  p.kv_bs = a.kv_bs;
  if (a.mode == SPATTEN_DECODE) return run_gemm<kQkvDecode>(p, a.dtype, stream);
  return run_gemm<kQkvPrefill>(p, a.dtype, stream);
}

int launch_out(const OutArgs& a, hipStream_t stream) {
  GemmParams p{};
  p.A = a.o;
  p.lda = int64_t(a.h_kept) * a.dh;
  p.W0 = a.wo;
  p.ldw = a.D;
  p.head_idx = a.head_idx;
  p.batch = a.batch;
  p.n = a.n;
  p.seq_tiled = a.h_kept != a.D / a.dh;
  p.M_total = a.batch * a.n;
  p.N = a.D;
  p.K = a.h_kept * a.dh;
  p.h_kept = a.h_kept;
  p.dh = a.dh;
  p.D = a.D;
  p.out0 = a.x;
  return run_gemm<kOut>(p, a.dtype, stream);
}

}  // namespace spatten
