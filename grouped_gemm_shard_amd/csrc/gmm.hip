// a6: grouped GEMM running the SwiGLU expert FFN over ragged groups.
//
// "Moe dynamic redundancy" (code review, rerouting comment) runs the local
// experts as one grouped matmul over their group sizes, redundant slots
// included; a replica slot computes with its home expert's weights.  The
// FFN itself is SwiGLU: act = SiLU(x Wg^T) * (x Wu^T), out = act Wd^T.
//
// bf16 path: two launches per pass.
//  * GEMM1 (x_sorted [N,H] against Wg and Wu [F,H]): a 128-row tile computes
//    128 act columns as 128 gate + 128 up columns held side by side in one
//    256-row weight tile, so the SwiGLU epilogue finds the gate and up value
//    of an element in the same lane and register.
//  * GEMM2 (act [N,F] against Wd [H,F]): a 128 x 256 output tile.
// Both use v_mfma_f32_32x32x16_bf16 with fp32 accumulation.  256 threads =
// 4 waves in a 2 x 2 grid, each wave a 64 x 128 slice = 2 x 4 MFMA tiles.
// K advances 64 per step through double-buffered LDS (rows padded to 72
// bf16 so that the 16-byte fragment reads of 32 consecutive rows spread
// over the banks); the next step's global loads are in flight while the
// current step's MFMAs run.
//
// Tiles: every group owns ceil(rows/128) m-tiles (an exclusive scan over
// groups, computed with the layout), so empty groups cost nothing; a block
// finds its group by binary search over the scan.
#include "common.h"

namespace moe {

namespace {

constexpr int BM = kGemmBM;  // 128
constexpr int BNB = 256;     // weight rows per tile
constexpr int BK = 64;
constexpr int LDK = BK + 8;  // padded LDS row (bf16 elements)

struct GemmParams {
  const uint16_t* A;
  const uint16_t* B0;  // gate weights (GEMM1) or down weights (GEMM2)
  const uint16_t* B1;  // up weights (GEMM1)
  size_t b_stride;     // elements per expert
  uint16_t* C;
  const int* group_offsets;
  const int* tile_off;
  const int* slot_expert;
  int G, K, Nout, lo_slot, e_base, e_res, n_ntiles;
  long long max_rows;
  PassArgs pa;
};

template <bool SWIGLU>
__global__ __launch_bounds__(256, 1) void gmm_bf16_kernel(GemmParams P) {
  PassInfo pi = resolve_pass(P.pa);
  if (!pi.active) return;
  const int total_mt = P.tile_off[P.G];
  if (P.group_offsets[P.G] > P.max_rows) return;  // malformed offsets: touch nothing
  const int mt = blockIdx.x / P.n_ntiles;
  const int nt = blockIdx.x - mt * P.n_ntiles;
  if (mt >= total_mt) return;
  int lo = 0, hi = P.G;
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (P.tile_off[mid] <= mt) lo = mid;
    else hi = mid;
  }
  const int g = lo;
  const int row0 = P.group_offsets[g] + (mt - P.tile_off[g]) * BM;
  const int rows = min(BM, P.group_offsets[g + 1] - row0);
  const int e = P.slot_expert[P.lo_slot + g] - P.e_base;
  if (e < 0 || e >= P.e_res) return;  // rows in a slot that hosts no resident expert

  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BNB * LDK];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w >> 1, wn = w & 1;

  const uint16_t* a_src[4];
  int a_dst[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int c = tid + i * 256, r = c >> 3, kc = c & 7;
    int rr = r < rows ? r : rows - 1;  // rows past the group repeat its last row
    a_src[i] = P.A + (size_t)(row0 + rr) * P.K + kc * 8;
    a_dst[i] = r * LDK + kc * 8;
  }
  const uint16_t* b_src[8];
  int b_dst[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    int c = tid + i * 256, r = c >> 3, kc = c & 7;
    const uint16_t* base;
    int wr;
    if (SWIGLU) {
      base = r < 128 ? P.B0 : P.B1;
      wr = nt * 128 + (r & 127);
    } else {
      base = P.B0;
      wr = nt * 256 + r;
    }
    b_src[i] = base + (size_t)e * P.b_stride + (size_t)wr * P.K + kc * 8;
    b_dst[i] = r * LDK + kc * 8;
  }

  uint4 ra[4], rb[8];
  floatx16 acc[2][4];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[mi][ni][q] = 0.0f;

  const int KT = P.K / BK;
#pragma unroll
  for (int i = 0; i < 4; ++i) ra[i] = *(const uint4*)(a_src[i]);
#pragma unroll
  for (int i = 0; i < 8; ++i) rb[i] = *(const uint4*)(b_src[i]);
#pragma unroll
  for (int i = 0; i < 4; ++i) *(uint4*)&As[0][a_dst[i]] = ra[i];
#pragma unroll
  for (int i = 0; i < 8; ++i) *(uint4*)&Bs[0][b_dst[i]] = rb[i];
  __syncthreads();

  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    const bool more = kt + 1 < KT;
    if (more) {
      const int k0 = (kt + 1) * BK;
#pragma unroll
      for (int i = 0; i < 4; ++i) ra[i] = *(const uint4*)(a_src[i] + k0);
#pragma unroll
      for (int i = 0; i < 8; ++i) rb[i] = *(const uint4*)(b_src[i] + k0);
    }
    const uint16_t* as = As[buf];
    const uint16_t* bs = Bs[buf];
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int kof = ks * 16 + (lane >> 5) * 8;
      bf16x8 a[2], b[4];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
        a[mi] = *(const bf16x8*)&as[(wm * 64 + mi * 32 + (lane & 31)) * LDK + kof];
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) {
        int brow = SWIGLU ? ((ni >> 1) * 128 + wn * 64 + (ni & 1) * 32) : (wn * 128 + ni * 32);
        b[ni] = *(const bf16x8*)&bs[(brow + (lane & 31)) * LDK + kof];
      }
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mi], b[ni], acc[mi][ni], 0, 0, 0);
    }
    if (more) {
#pragma unroll
      for (int i = 0; i < 4; ++i) *(uint4*)&As[buf ^ 1][a_dst[i]] = ra[i];
#pragma unroll
      for (int i = 0; i < 8; ++i) *(uint4*)&Bs[buf ^ 1][b_dst[i]] = rb[i];
    }
    __syncthreads();
  }

  // 32x32 accumulator layout: register q of a lane holds row
  // (q/4)*8 + (lane/32)*4 + q%4, column lane%32.
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int lr = wm * 64 + mi * 32 + (q >> 2) * 8 + (lane >> 5) * 4 + (q & 3);
      if (lr >= rows) continue;
      uint16_t* crow = P.C + (size_t)(row0 + lr) * P.Nout;
      if (SWIGLU) {
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
          float gv = acc[mi][ni][q], uv = acc[mi][ni + 2][q];
          float av = gv / (1.0f + __expf(-gv)) * uv;
          crow[nt * 128 + wn * 64 + ni * 32 + (lane & 31)] = f2bf(av);
        }
      } else {
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
          crow[nt * 256 + wn * 128 + ni * 32 + (lane & 31)] = f2bf(acc[mi][ni][q]);
      }
    }
  }
}

// fp32 path (the tiny fp32 workload): one thread per output element.
struct F32Params {
  const float* A;
  const float* B0;
  const float* B1;
  size_t b_stride;
  float* C;
  const int* group_offsets;
  const int* slot_expert;
  int G, K, Nout, lo_slot, e_base, e_res;
  long long max_rows;
  PassArgs pa;
};

template <bool SWIGLU>
__global__ __launch_bounds__(256) void gmm_f32_kernel(F32Params P) {
  PassInfo pi = resolve_pass(P.pa);
  if (!pi.active) return;
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const int row = (int)(idx / P.Nout), col = (int)(idx - (long long)row * P.Nout);
  if (row >= P.group_offsets[P.G] || P.group_offsets[P.G] > P.max_rows) return;
  int lo = 0, hi = P.G;
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (P.group_offsets[mid] <= row) lo = mid;
    else hi = mid;
  }
  const int e = P.slot_expert[P.lo_slot + lo] - P.e_base;
  if (e < 0 || e >= P.e_res) return;
  const float* a = P.A + (size_t)row * P.K;
  const float* w0 = P.B0 + (size_t)e * P.b_stride + (size_t)col * P.K;
  float s0 = 0.0f, s1 = 0.0f;
  if (SWIGLU) {
    const float* w1 = P.B1 + (size_t)e * P.b_stride + (size_t)col * P.K;
    for (int kk = 0; kk < P.K; ++kk) {
      s0 = fmaf(a[kk], w0[kk], s0);
      s1 = fmaf(a[kk], w1[kk], s1);
    }
    P.C[(size_t)row * P.Nout + col] = s0 / (1.0f + __expf(-s0)) * s1;
  } else {
    for (int kk = 0; kk < P.K; ++kk) s0 = fmaf(a[kk], w0[kk], s0);
    P.C[(size_t)row * P.Nout + col] = s0;
  }
}

// m-tile offsets from group offsets (standalone grouped GEMM calls).
__global__ __launch_bounds__(1024) void tile_schedule_kernel(int G, const int* group_offsets,
                                                             int* tile_off, PassArgs pa) {
  PassInfo pi = resolve_pass(pa);
  if (!pi.active) return;
  __shared__ int tmp[16];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  int g = threadIdx.x;
  int v = g < G ? (group_offsets[g + 1] - group_offsets[g] + BM - 1) / BM : 0;
  int x = v;
  for (int off = 1; off < 64; off <<= 1) {
    int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) tmp[w] = x;
  __syncthreads();
  if (w == 0) {
    int t = lane < nw ? tmp[lane] : 0;
    for (int off = 1; off < 64; off <<= 1) {
      int y = __shfl_up(t, off);
      if (lane >= off) t += y;
    }
    if (lane < nw) tmp[lane] = t;
  }
  __syncthreads();
  int ex = (w > 0 ? tmp[w - 1] : 0) + x - v;
  if (g < G) tile_off[g] = ex;
  if (g == 0) tile_off[G] = tmp[nw - 1];
}

}  // namespace

size_t gmm_scratch_bytes(const Dims& d) { return ((size_t)(d.G_res + 1) * 4 + 255) / 256 * 256; }

hipError_t launch_gmm(const Dims& d, const PassArgs& pa, const void* x_sorted,
                      const int* group_offsets, const int* tile_off, const int* slot_expert,
                      const void* wg, const void* wu, const void* wd, void* act, void* out,
                      int64_t max_rows, void* scratch, hipStream_t s) {
  if (d.bf16) {
    int* toff = (int*)tile_off;
    if (toff == nullptr) {
      toff = (int*)scratch;
      hipLaunchKernelGGL(tile_schedule_kernel, dim3(1), dim3(1024), 0, s, d.G_res, group_offsets,
                         toff, pa);
    }
    const long long mt_ub = (max_rows + BM - 1) / BM + d.G_res;
    GemmParams p1;
    p1.A = (const uint16_t*)x_sorted;
    p1.B0 = (const uint16_t*)wg;
    p1.B1 = (const uint16_t*)wu;
    p1.b_stride = (size_t)d.F * d.H;
    p1.C = (uint16_t*)act;
    p1.group_offsets = group_offsets;
    p1.tile_off = toff;
    p1.slot_expert = slot_expert;
    p1.G = d.G_res;
    p1.K = d.H;
    p1.Nout = d.F;
    p1.lo_slot = d.lo_slot;
    p1.e_base = d.e_base;
    p1.e_res = d.S_res * d.El;
    p1.max_rows = max_rows;
    p1.n_ntiles = d.F / 128;
    p1.pa = pa;
    hipLaunchKernelGGL(gmm_bf16_kernel<true>, dim3((unsigned)(mt_ub * p1.n_ntiles)), dim3(256), 0,
                       s, p1);
    GemmParams p2 = p1;
    p2.A = (const uint16_t*)act;
    p2.B0 = (const uint16_t*)wd;
    p2.B1 = nullptr;
    p2.b_stride = (size_t)d.H * d.F;
    p2.C = (uint16_t*)out;
    p2.K = d.F;
    p2.Nout = d.H;
    p2.n_ntiles = d.H / 256;
    hipLaunchKernelGGL(gmm_bf16_kernel<false>, dim3((unsigned)(mt_ub * p2.n_ntiles)), dim3(256),
                       0, s, p2);
  } else {
    F32Params p1;
    p1.A = (const float*)x_sorted;
    p1.B0 = (const float*)wg;
    p1.B1 = (const float*)wu;
    p1.b_stride = (size_t)d.F * d.H;
    p1.C = (float*)act;
    p1.group_offsets = group_offsets;
    p1.slot_expert = slot_expert;
    p1.G = d.G_res;
    p1.K = d.H;
    p1.Nout = d.F;
    p1.lo_slot = d.lo_slot;
    p1.e_base = d.e_base;
    p1.e_res = d.S_res * d.El;
    p1.max_rows = max_rows;
    p1.pa = pa;
    long long n1 = max_rows * (long long)d.F;
    hipLaunchKernelGGL(gmm_f32_kernel<true>, dim3((unsigned)((n1 + 255) / 256)), dim3(256), 0, s,
                       p1);
    F32Params p2 = p1;
    p2.A = (const float*)act;
    p2.B0 = (const float*)wd;
    p2.B1 = nullptr;
    p2.b_stride = (size_t)d.H * d.F;
    p2.C = (float*)out;
    p2.K = d.F;
    p2.Nout = d.H;
    long long n2 = max_rows * (long long)d.H;
    hipLaunchKernelGGL(gmm_f32_kernel<false>, dim3((unsigned)((n2 + 255) / 256)), dim3(256), 0,
                       s, p2);
  }
  return hipGetLastError();
}

}  // namespace moe
