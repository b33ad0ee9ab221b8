// Backward of the one-shard MoE layer.
//
// "Support moe_dropless_fallback=layer on the ragged all-to-all MoE path"
// (How) runs the chunked passes in a scan whose backward recomputes one
// chunk at a time and carries the weight gradients across the chunks; "MoE
// ring-of-experts: TC Pallas ring all-gather for the combine backward +
// x_sorted remat save" (What) keeps the expert-sorted input x_sorted for
// the backward.  The steps here are the chain rule of the forward ones:
//
//  * combine backward: d_out[row(t,j)] = g_tj dy_t and d_gate[t,j] =
//    <dy_t, out[row(t,j)]>, one wave per token;
//  * grouped GEMM backward (bf16, MFMA): with h_g = x Wg^T, h_u = x Wu^T,
//      d_a  = d_out Wd                          (GEMM, K = H, against Wd^T)
//      d_hg = d_a h_u SiLU'(h_g), d_hu = d_a SiLU(h_g), a = SiLU(h_g) h_u
//           (the forward's GEMM1 recomputed, SwiGLU backward in its epilogue)
//      dx_sorted = [d_hg | d_hu] [Wg ; Wu]      (GEMM, K = 2F, against
//                                                [Wg ; Wu]^T)
//      [dWg ; dWu] = [d_hg | d_hu]^T x_sorted,  dWd = d_out^T a
//                                               (reductions over each
//                                                expert's ragged rows)
//    The data-gradient GEMMs read the weights transposed (K contiguous),
//    made once per weight update by moe_transpose_weights; the
//    weight-gradient GEMMs reduce over rows, so their operands are
//    transposed on the way into LDS;
//  * permute backward: dx_t = the sum of dx_sorted over the token's rows,
//    one wave per token;
//  * gate backward into the logits, one wave per token.
#include "common.h"

namespace moe {

namespace {

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// 16-byte vectors of the activation dtype as 8 (bf16) or 4 (fp32) floats.
template <bool BF16>
struct Vec {
  static constexpr int N = BF16 ? 8 : 4;
  float v[N];
  __device__ __forceinline__ void load(const void* base, size_t elem) {
    const uint4 u = *(const uint4*)((const char*)base + elem * (BF16 ? 2 : 4));
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
    if (BF16) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = __uint_as_float(w[i]);
    }
  }
  __device__ __forceinline__ void store(void* base, size_t elem) const {
    uint32_t w[4];
    if (BF16) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        w[i] = (uint32_t)f2bf(v[2 * i]) | ((uint32_t)f2bf(v[2 * i + 1]) << 16);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = __float_as_uint(v[i]);
    }
    *(uint4*)((char*)base + elem * (BF16 ? 2 : 4)) = make_uint4(w[0], w[1], w[2], w[3]);
  }
};

// ---- combine backward ------------------------------------------------------

template <bool BF16>
__global__ __launch_bounds__(256) void combine_bwd_kernel(Dims d, PassArgs pa, const void* dy,
                                                          const void* out, const int* roa,
                                                          const float* gate, void* d_out,
                                                          float* d_gate, long long max_rows) {
  const PassInfo pi = resolve_pass(pa);
  if (!pi.active) return;
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (i >= pass_tokens(d, pi)) return;
  const int t = pass_token(d, pi, i);
  const int lane = threadIdx.x & 63;
  constexpr int N = Vec<BF16>::N;
  for (int j = 0; j < d.k; ++j) {
    const int r = roa[(size_t)t * d.k + j];
    float dot = 0.0f;
    if (r >= 0 && r < max_rows) {
      const float g = gate[(size_t)t * d.k + j];
      for (int c = lane * N; c < d.H; c += 64 * N) {
        Vec<BF16> a, o;
        a.load(dy, (size_t)t * d.H + c);
        o.load(out, (size_t)r * d.H + c);
#pragma unroll
        for (int q = 0; q < N; ++q) {
          dot = fmaf(a.v[q], o.v[q], dot);
          a.v[q] *= g;
        }
        a.store(d_out, (size_t)r * d.H + c);
      }
    }
    dot = wave_sum(dot);
    if (lane == 0) d_gate[(size_t)t * d.k + j] = dot;
  }
}

// ---- permute backward ------------------------------------------------------

template <bool BF16>
__global__ __launch_bounds__(256) void permute_bwd_kernel(Dims d, PassArgs pa, const void* dxs,
                                                          const int* roa, void* dx,
                                                          long long max_rows) {
  const PassInfo pi = resolve_pass(pa);
  if (!pi.active) return;
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (i >= pass_tokens(d, pi)) return;
  const int t = pass_token(d, pi, i);
  const int lane = threadIdx.x & 63;
  constexpr int N = Vec<BF16>::N;
  for (int c = lane * N; c < d.H; c += 64 * N) {
    Vec<BF16> acc;
#pragma unroll
    for (int q = 0; q < N; ++q) acc.v[q] = 0.0f;
    for (int j = 0; j < d.k; ++j) {
      const int r = roa[(size_t)t * d.k + j];
      if (r < 0 || r >= max_rows) continue;
      Vec<BF16> v;
      v.load(dxs, (size_t)r * d.H + c);
#pragma unroll
      for (int q = 0; q < N; ++q) acc.v[q] += v.v[q];
    }
    acc.store(dx, (size_t)t * d.H + c);
  }
}

// ---- gate backward ---------------------------------------------------------

__global__ __launch_bounds__(256) void route_bwd_kernel(Dims d, const int* idx, const float* gate,
                                                        const float* d_gate, float* d_logits) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= d.T) return;
  const int lane = threadIdx.x & 63;
  float g = 0.0f, dg = 0.0f;
  int e = -1;
  if (lane < d.k) {
    g = gate[(size_t)t * d.k + lane];
    dg = d_gate[(size_t)t * d.k + lane];
    e = idx[(size_t)t * d.k + lane];
  }
  float v;
  if (d.gate == MOE_GATE_SOFTMAX) {
    const float s = wave_sum(g * dg);
    v = g * (dg - s);
  } else {
    v = dg * g * (1.0f - g);
  }
  for (int c = lane; c < d.E; c += 64) {
    float o = 0.0f;
    for (int j = 0; j < d.k; ++j) {
      const int ej = __shfl(e, j);
      const float vj = __shfl(v, j);
      if (ej == c) o += vj;
    }
    d_logits[(size_t)t * d.E + c] = o;
  }
}

// ---- weight transposes -----------------------------------------------------

// out[e][c][col0 + r] = in[e][r][c] for 64 x 64 tiles (R, C multiples of 64).
__global__ __launch_bounds__(256) void transpose_kernel(const uint16_t* in, uint16_t* out, int R,
                                                        int C, long long in_e, long long out_e,
                                                        int ldo, int col0) {
  __shared__ uint16_t tile[64][66];
  const int ct = blockIdx.x, rt = blockIdx.y, e = blockIdx.z;
  const uint16_t* src = in + (size_t)e * in_e + (size_t)rt * 64 * C + (size_t)ct * 64;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
  for (int r = ty; r < 64; r += 8) {
    const uint32_t w = *(const uint32_t*)(src + (size_t)r * C + tx * 2);
    tile[r][tx * 2] = (uint16_t)(w & 0xFFFF);
    tile[r][tx * 2 + 1] = (uint16_t)(w >> 16);
  }
  __syncthreads();
  uint16_t* dst = out + (size_t)e * out_e + (size_t)ct * 64 * ldo + col0 + (size_t)rt * 64;
  for (int c = ty; c < 64; c += 8) {
    const uint32_t w = (uint32_t)tile[tx * 2][c] | ((uint32_t)tile[tx * 2 + 1][c] << 16);
    *(uint32_t*)(dst + (size_t)c * ldo + tx * 2) = w;
  }
}

// ---- m-tiles of the data-gradient GEMMs ------------------------------------

constexpr int kBM = 128;  // rows per tile
constexpr int kBN = 128;  // output columns per tile
constexpr int kBK = 32;   // reduction columns per stage
constexpr int kNST = 3;   // ring stages

// tile_off[g] = m-tiles of groups before g (kBM rows each); offsets that are
// not non-decreasing within [0, limit] give no tiles.
__global__ __launch_bounds__(1024) void bwd_tiles_kernel(int G, int limit,
                                                         const int* group_offsets,
                                                         int* tile_off) {
  __shared__ int wsum[16];
  __shared__ int bad;
  if (threadIdx.x == 0) bad = 0;
  __syncthreads();
  const int g = threadIdx.x, lane = g & 63, w = g >> 6;
  int v = 0;
  if (g < G) {
    const int a = group_offsets[g], b = group_offsets[g + 1];
    if (a < 0 || b < a || b > limit) bad = 1;
    v = (b - a + kBM - 1) / kBM;
  }
  __syncthreads();
  if (bad) v = 0;
  int x = v;
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  int base = 0;
  for (int i = 0; i < w; ++i) base += wsum[i];
  if (g < G) tile_off[g] = base + x - v;
  if (g == 0) {
    int tot = 0;
    for (int i = 0; i < 16; ++i) tot += wsum[i];
    tile_off[G] = tot;
  }
}

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void* base, unsigned bytes) {
  // loads at offsets >= bytes return zero
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// 16-byte chunk permutation of a 64-byte LDS row (4 chunks): fragment reads
// of consecutive rows at one chunk land on distinct banks.
__device__ __forceinline__ int swz4(int row) { return (row >> 2) & 3; }

template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

struct DgradParams {
  const uint16_t* A;        // [a_rows, K] rows of the pass
  int a_rows;
  const uint16_t* B0;       // [e_res][Nout][K] (SwiGLU: gate weights)
  const uint16_t* B1;       // SwiGLU: up weights
  size_t b_stride;
  uint16_t* C;              // plain: [rows, Nout]
  const uint16_t* d_a;      // SwiGLU backward: [rows, Nout]
  uint16_t* d_h;            // SwiGLU backward: [rows, 2 Nout] (d_hg | d_hu)
  uint16_t* act;            // SwiGLU backward: [rows, Nout] recomputed activation
  const int* group_offsets;
  const int* tile_off;
  const int* slot_expert;
  int G, K, Nout, lo_slot, e_base, e_res, n_ntiles;
  long long max_rows;
};

// One 128 x 128 output tile of group rows (plain: C = A B^T; SwiGLU
// backward: the gate and up products of 128 activation columns, 256 weight
// rows).  4 waves in a 2 x 2 grid, 64 x 64 per wave, v_mfma 32x32x16 bf16;
// operands stream from HBM into a 3-stage LDS ring with buffer_load ... lds.
template <bool SW>
__device__ __forceinline__ void dgrad_tile(const DgradParams& P) {
  constexpr int RB = kBK * 2;                  // 64 bytes per row per stage
  constexpr int CPR = kBK / 8;                 // 4 chunks per row
  constexpr int RPI = 1024 / RB;               // 16 rows per wave-wide load
  constexpr int BROWS = SW ? 2 * kBN : kBN;    // weight rows per tile
  constexpr int AI = kBM / RPI / 4, BI = BROWS / RPI / 4;
  constexpr int LPS = AI + BI;
  constexpr int SA = kBM * RB, SS = (kBM + BROWS) * RB;
  constexpr int NS = 2;                        // acc sets (gate, up) or 1
  __shared__ __attribute__((aligned(1024))) char smem[kNST * SS];

  const int nt = blockIdx.x % P.n_ntiles;
  const int m = blockIdx.x / P.n_ntiles;
  const int total = P.tile_off[P.G];
  if (m >= total) return;
  int lo = 0, hi = P.G;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (P.tile_off[mid] <= m) lo = mid;
    else hi = mid;
  }
  const int g = lo;
  const int gend = P.group_offsets[g + 1];
  const int row0 = P.group_offsets[g] + (m - P.tile_off[g]) * kBM;
  if (row0 < 0 || row0 >= gend || gend > P.max_rows) return;
  const int rows = min(kBM, gend - row0);
  const int e = P.slot_expert[P.lo_slot + g] - P.e_base;
  if (e < 0 || e >= P.e_res) return;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int K = P.K, KT = K / kBK;
  const __amdgpu_buffer_rsrc_t ra = raw_rsrc(P.A, (unsigned)P.a_rows * K * 2);
  const size_t boff = (size_t)e * P.b_stride + (size_t)nt * kBN * K;
  const __amdgpu_buffer_rsrc_t rb0 = raw_rsrc(P.B0 + boff, (unsigned)kBN * K * 2);
  const __amdgpu_buffer_rsrc_t rb1 = SW ? raw_rsrc(P.B1 + boff, (unsigned)kBN * K * 2) : rb0;
  int a_off[AI], b_off[BI];
#pragma unroll
  for (int i = 0; i < AI; ++i) {
    const int row = (i * 4 + w) * RPI + lane / CPR;
    a_off[i] = row < rows ? (row0 + row) * K * 2 + (((lane % CPR) ^ swz4(row)) << 4)
                          : (int)0x80000000;
  }
#pragma unroll
  for (int i = 0; i < BI; ++i) {
    const int row = (i * 4 + w) * RPI + lane / CPR;
    b_off[i] = (row % kBN) * K * 2 + (((lane % CPR) ^ swz4(row)) << 4);
  }
  auto issue = [&](int step) {
    char* st = smem + (step % kNST) * SS;
    const int kb = step * kBK * 2;
#pragma unroll
    for (int i = 0; i < AI; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(st + (i * 4 + w) * RPI * RB), 16,
                                               a_off[i], kb, 0, 0);
#pragma unroll
    for (int i = 0; i < BI; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(SW && i >= BI / 2 ? rb1 : rb0,
                                               (lds_void*)(st + SA + (i * 4 + w) * RPI * RB), 16,
                                               b_off[i], kb, 0, 0);
  };

  floatx16 acc[SW ? NS : 1][2][2];
#pragma unroll
  for (int s = 0; s < (SW ? NS : 1); ++s)
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[s][mi][ni][q] = 0.0f;

  int a_row[2], b_row[2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) a_row[mi] = wm * 64 + mi * 32 + (lane & 31);
#pragma unroll
  for (int ni = 0; ni < 2; ++ni) b_row[ni] = wn * 64 + ni * 32 + (lane & 31);

#pragma unroll
  for (int s = 0; s < kNST - 1; ++s)
    if (s < KT) issue(s);
  for (int kt = 0; kt < KT; ++kt) {
    if (kt + 1 < KT) wait_vm_barrier<LPS>();
    else wait_vm_barrier<0>();
    if (kt + kNST - 1 < KT) issue(kt + kNST - 1);
    const char* sa = smem + (kt % kNST) * SS;
    const char* sb = sa + SA;
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      const int kc = ks * 2 + (lane >> 5);
      bf16x8 a[2], b[SW ? 2 : 1][2];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
        a[mi] = *(const bf16x8*)(sa + a_row[mi] * RB + ((kc ^ swz4(a_row[mi])) << 4));
#pragma unroll
      for (int s = 0; s < (SW ? 2 : 1); ++s)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
          const int br = s * kBN + b_row[ni];
          b[s][ni] = *(const bf16x8*)(sb + br * RB + ((kc ^ swz4(br)) << 4));
        }
#pragma unroll
      for (int s = 0; s < (SW ? 2 : 1); ++s)
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
          for (int ni = 0; ni < 2; ++ni)
            acc[s][mi][ni] =
                __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mi], b[s][ni], acc[s][mi][ni], 0, 0, 0);
    }
  }

  // Epilogue: 32x32 accumulator layout, register q of a lane holds row
  // (q/4)*8 + (lane/32)*4 + q%4 and column lane%32 of its MFMA tile.
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int lr = wm * 64 + mi * 32 + (q >> 2) * 8 + (lane >> 5) * 4 + (q & 3);
      if (lr >= rows) continue;
      const size_t r = (size_t)(row0 + lr);
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        const int c = nt * kBN + wn * 64 + ni * 32 + (lane & 31);
        if (SW) {
          const float gv = acc[0][mi][ni][q], uv = acc[SW ? 1 : 0][mi][ni][q];
          const float da = bf2f(P.d_a[r * P.Nout + c]);
          // the forward's SiLU with the hardware reciprocal
          const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-gv));
          const float silu = gv * sg;
          P.act[r * P.Nout + c] = f2bf(silu * uv);
          P.d_h[r * 2 * P.Nout + c] = f2bf(da * uv * (sg * (1.0f + gv * (1.0f - sg))));
          P.d_h[r * 2 * P.Nout + P.Nout + c] = f2bf(da * silu);
        } else {
          P.C[r * P.Nout + c] = f2bf(acc[0][mi][ni][q]);
        }
      }
    }
}

template <bool SW>
__global__ __launch_bounds__(256, 2) void dgrad_kernel(DgradParams P) {
  dgrad_tile<SW>(P);
}

// ---- weight-gradient GEMM --------------------------------------------------

struct WgradParams {
  const uint16_t* Pm;   // [rows, I] (row-major, I contiguous)
  const uint16_t* Qm;   // [rows, J]
  float* C0;            // rows i < i_split: C0[e][i][j]
  float* C1;            // rows i >= i_split: C1[e][i - i_split][j]
  size_t c_stride;      // elements per expert of C0 / C1
  int I, J, i_split;
  const int* group_offsets;
  const int* slot_expert;
  int G, lo_slot, e_base, e_res, ni_tiles, nj_tiles;
  long long max_rows;
  int accumulate;
};

// Next (group, row) step of expert e's rows after (g, r): the rows of its
// groups in group order, 32 at a time.  g = G when there are none left.
__device__ __forceinline__ void wgrad_next(const WgradParams& P, int e, int& g, int& r) {
  r += kBK;
  if (g >= 0 && g < P.G && r < P.group_offsets[g + 1]) return;
  for (++g; g < P.G; ++g) {
    if (P.slot_expert[P.lo_slot + g] - P.e_base != e) continue;
    const int a = P.group_offsets[g], b = P.group_offsets[g + 1];
    if (b > a && b <= P.max_rows && a >= 0) {
      r = a;
      return;
    }
  }
}

// One 128 x 128 tile of C[e] = P^T Q over expert e's rows.  4 waves in a
// 2 x 2 grid, 64 x 64 per wave.  Each step stages 32 rows of both operands:
// a thread loads one 4-byte pair of columns from 8 consecutive rows and
// writes them to LDS as two 16-byte runs of 8 rows (row index contiguous),
// so the MFMA fragments read 8 consecutive reduction elements at once.
// Double-buffered: the next step's loads are in flight during the MFMAs.
__global__ __launch_bounds__(256, 2) void wgrad_kernel(WgradParams P) {
  constexpr int RB = kBK * 2;  // 64 bytes: one operand column's 32 rows
  constexpr int TS = 128 * RB;  // one operand tile
  __shared__ __attribute__((aligned(1024))) char smem[2][2 * TS];
  const int per_e = P.ni_tiles * P.nj_tiles;
  const int e = blockIdx.x / per_e;
  const int it = (blockIdx.x % per_e) / P.nj_tiles, jt = blockIdx.x % P.nj_tiles;
  if (e >= P.e_res) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int i0 = it * 128, j0 = jt * 128;

  int g = -1, r = -kBK;
  wgrad_next(P, e, g, r);
  int gend = g < P.G ? P.group_offsets[g + 1] : 0;

  uint32_t pv[8], qv[8];
  auto load = [&](int gr, int rr, int ge) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int row = rr + w * 8 + q;
      if (gr < P.G && row < ge) {
        pv[q] = *(const uint32_t*)(P.Pm + (size_t)row * P.I + i0 + lane * 2);
        qv[q] = *(const uint32_t*)(P.Qm + (size_t)row * P.J + j0 + lane * 2);
      } else {
        pv[q] = 0u;
        qv[q] = 0u;
      }
    }
  };
  // columns 2*lane and 2*lane+1, rows w*8 .. w*8+7 of the step
  auto stage = [&](char* buf) {
#pragma unroll
    for (int op = 0; op < 2; ++op) {
      const uint32_t* v = op == 0 ? pv : qv;
      uint4 lo4, hi4;
      lo4.x = (v[0] & 0xFFFFu) | (v[1] << 16);
      lo4.y = (v[2] & 0xFFFFu) | (v[3] << 16);
      lo4.z = (v[4] & 0xFFFFu) | (v[5] << 16);
      lo4.w = (v[6] & 0xFFFFu) | (v[7] << 16);
      hi4.x = (v[0] >> 16) | (v[1] & 0xFFFF0000u);
      hi4.y = (v[2] >> 16) | (v[3] & 0xFFFF0000u);
      hi4.z = (v[4] >> 16) | (v[5] & 0xFFFF0000u);
      hi4.w = (v[6] >> 16) | (v[7] & 0xFFFF0000u);
      char* t = buf + op * TS;
      const int c0 = lane * 2, c1 = lane * 2 + 1;
      *(uint4*)(t + c0 * RB + ((w ^ swz4(c0)) << 4)) = lo4;
      *(uint4*)(t + c1 * RB + ((w ^ swz4(c1)) << 4)) = hi4;
    }
  };

  floatx16 acc[2][2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[mi][ni][q] = 0.0f;

  int cur = 0;
  if (g < P.G) {
    load(g, r, gend);
    stage(smem[0]);
  }
  __syncthreads();
  while (g < P.G) {
    int g2 = g, r2 = r;
    wgrad_next(P, e, g2, r2);
    const int gend2 = g2 < P.G ? P.group_offsets[g2 + 1] : 0;
    if (g2 < P.G) load(g2, r2, gend2);
    const char* sp = smem[cur];
    const char* sq = sp + TS;
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      const int kc = ks * 2 + (lane >> 5);
      bf16x8 a[2], b[2];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) {
        const int row = wm * 64 + mi * 32 + (lane & 31);
        a[mi] = *(const bf16x8*)(sp + row * RB + ((kc ^ swz4(row)) << 4));
      }
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        const int row = wn * 64 + ni * 32 + (lane & 31);
        b[ni] = *(const bf16x8*)(sq + row * RB + ((kc ^ swz4(row)) << 4));
      }
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mi], b[ni], acc[mi][ni], 0, 0, 0);
    }
    if (g2 < P.G) stage(smem[cur ^ 1]);
    __syncthreads();
    cur ^= 1;
    g = g2;
    r = r2;
    gend = gend2;
  }

#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int i = i0 + wm * 64 + mi * 32 + (q >> 2) * 8 + (lane >> 5) * 4 + (q & 3);
      float* crow = i < P.i_split ? P.C0 + (size_t)e * P.c_stride + (size_t)i * P.J
                                  : P.C1 + (size_t)e * P.c_stride + (size_t)(i - P.i_split) * P.J;
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        const int j = j0 + wn * 64 + ni * 32 + (lane & 31);
        const float v = acc[mi][ni][q];
        crow[j] = P.accumulate ? crow[j] + v : v;
      }
    }
}

// ---- fp32 path (small fp32 problems): one thread per output element -------

struct F32Bwd {
  const float* x;       // x_sorted [rows, H]
  const float* wg;      // [e_res, F, H]
  const float* wu;
  const float* wd;      // [e_res, H, F]
  const float* d_out;   // [rows, H]
  float* d_h;           // [rows, 2F]
  float* act;           // [rows, F]
  float* dxs;           // [rows, H]
  float* dwg;
  float* dwu;
  float* dwd;
  const int* group_offsets;
  const int* slot_expert;
  int G, H, F, lo_slot, e_base, e_res;
  long long max_rows;
  int accumulate;
};

__device__ __forceinline__ int f32_group(const F32Bwd& P, int row) {
  int lo = 0, hi = P.G;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (P.group_offsets[mid] <= row) lo = mid;
    else hi = mid;
  }
  return lo;
}

// d_h and act for (row, f): the gate and up products recomputed, d_a from Wd.
__global__ __launch_bounds__(256) void f32_dh_kernel(F32Bwd P) {
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const int row = (int)(idx / P.F), f = (int)(idx % P.F);
  const int n = P.group_offsets[P.G];
  if (row >= n || n > P.max_rows) return;
  const int e = P.slot_expert[P.lo_slot + f32_group(P, row)] - P.e_base;
  if (e < 0 || e >= P.e_res) return;
  const float* xr = P.x + (size_t)row * P.H;
  const float* g = P.wg + ((size_t)e * P.F + f) * P.H;
  const float* u = P.wu + ((size_t)e * P.F + f) * P.H;
  const float* dor = P.d_out + (size_t)row * P.H;
  const float* wd = P.wd + (size_t)e * P.H * P.F + f;
  float hg = 0.0f, hu = 0.0f, da = 0.0f;
  for (int h = 0; h < P.H; ++h) {
    hg = fmaf(xr[h], g[h], hg);
    hu = fmaf(xr[h], u[h], hu);
    da = fmaf(dor[h], wd[(size_t)h * P.F], da);
  }
  const float sg = 1.0f / (1.0f + __expf(-hg));
  const float silu = hg * sg;
  P.act[(size_t)row * P.F + f] = silu * hu;
  P.d_h[(size_t)row * 2 * P.F + f] = da * hu * (sg * (1.0f + hg * (1.0f - sg)));
  P.d_h[(size_t)row * 2 * P.F + P.F + f] = da * silu;
}

__global__ __launch_bounds__(256) void f32_dx_kernel(F32Bwd P) {
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const int row = (int)(idx / P.H), h = (int)(idx % P.H);
  const int n = P.group_offsets[P.G];
  if (row >= n || n > P.max_rows) return;
  const int e = P.slot_expert[P.lo_slot + f32_group(P, row)] - P.e_base;
  if (e < 0 || e >= P.e_res) return;
  const float* dh = P.d_h + (size_t)row * 2 * P.F;
  const float* g = P.wg + (size_t)e * P.F * P.H + h;
  const float* u = P.wu + (size_t)e * P.F * P.H + h;
  float s = 0.0f;
  for (int f = 0; f < P.F; ++f) {
    s = fmaf(dh[f], g[(size_t)f * P.H], s);
    s = fmaf(dh[P.F + f], u[(size_t)f * P.H], s);
  }
  P.dxs[(size_t)row * P.H + h] = s;
}

// which: 0 = dWg [F,H], 1 = dWu [F,H], 2 = dWd [H,F]; one thread per element
// of one expert's gradient, summing the expert's rows in group order.
__global__ __launch_bounds__(256) void f32_dw_kernel(F32Bwd P, int which) {
  const long long per = (long long)P.F * P.H;
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const int e = (int)(idx / per);
  if (e >= P.e_res) return;
  const long long o = idx % per;
  const int a = (int)(o / (which == 2 ? P.F : P.H)), b = (int)(o % (which == 2 ? P.F : P.H));
  float s = 0.0f;
  for (int g = 0; g < P.G; ++g) {
    if (P.slot_expert[P.lo_slot + g] - P.e_base != e) continue;
    const int r0 = P.group_offsets[g], r1 = P.group_offsets[g + 1];
    if (r0 < 0 || r1 > P.max_rows) continue;
    for (int r = r0; r < r1; ++r) {
      if (which == 2)
        s = fmaf(P.d_out[(size_t)r * P.H + a], P.act[(size_t)r * P.F + b], s);
      else
        s = fmaf(P.d_h[(size_t)r * 2 * P.F + which * P.F + a], P.x[(size_t)r * P.H + b], s);
    }
  }
  float* dst = which == 0 ? P.dwg : which == 1 ? P.dwu : P.dwd;
  dst[idx] = P.accumulate ? dst[idx] + s : s;
}

inline size_t a256(size_t b) { return (b + 255) / 256 * 256; }

}  // namespace

size_t gmm_bwd_scratch_bytes(const Dims& d, int64_t max_rows) {
  const size_t el = d.bf16 ? 2 : 4;
  return a256((size_t)(d.G_res + 1) * 4) + 3 * a256((size_t)max_rows * d.F * el) +
         a256((size_t)max_rows * d.F * el);
}

hipError_t launch_transpose_weights(const Dims& d, const void* wg, const void* wu,
                                    const void* wd, void* wgu_t, void* wd_t, hipStream_t s) {
  const int e_res = d.S_res * d.El;
  // [E,F,H] gate / up -> [E,H,2F] (gate in columns [0,F), up in [F,2F))
  hipLaunchKernelGGL(transpose_kernel, dim3(d.H / 64, d.F / 64, e_res), dim3(256), 0, s,
                     (const uint16_t*)wg, (uint16_t*)wgu_t, d.F, d.H, (long long)d.F * d.H,
                     (long long)d.H * 2 * d.F, 2 * d.F, 0);
  hipLaunchKernelGGL(transpose_kernel, dim3(d.H / 64, d.F / 64, e_res), dim3(256), 0, s,
                     (const uint16_t*)wu, (uint16_t*)wgu_t, d.F, d.H, (long long)d.F * d.H,
                     (long long)d.H * 2 * d.F, 2 * d.F, d.F);
  // [E,H,F] down -> [E,F,H]
  hipLaunchKernelGGL(transpose_kernel, dim3(d.F / 64, d.H / 64, e_res), dim3(256), 0, s,
                     (const uint16_t*)wd, (uint16_t*)wd_t, d.H, d.F, (long long)d.H * d.F,
                     (long long)d.F * d.H, d.H, 0);
  return hipGetLastError();
}

hipError_t launch_combine_bwd(const Dims& d, const PassArgs& pa, const void* dy,
                              const void* out, const int* roa, const float* gate, void* d_out,
                              float* d_gate, int64_t max_rows, hipStream_t s) {
  const int ntok = (d.T / d.L) * pa.lw;
  const dim3 grid((ntok + 3) / 4);
  if (d.bf16)
    hipLaunchKernelGGL(combine_bwd_kernel<true>, grid, dim3(256), 0, s, d, pa, dy, out, roa, gate,
                       d_out, d_gate, (long long)max_rows);
  else
    hipLaunchKernelGGL(combine_bwd_kernel<false>, grid, dim3(256), 0, s, d, pa, dy, out, roa,
                       gate, d_out, d_gate, (long long)max_rows);
  return hipGetLastError();
}

hipError_t launch_permute_bwd(const Dims& d, const PassArgs& pa, const void* dxs,
                              const int* roa, void* dx, int64_t max_rows, hipStream_t s) {
  const int ntok = (d.T / d.L) * pa.lw;
  const dim3 grid((ntok + 3) / 4);
  if (d.bf16)
    hipLaunchKernelGGL(permute_bwd_kernel<true>, grid, dim3(256), 0, s, d, pa, dxs, roa, dx,
                       (long long)max_rows);
  else
    hipLaunchKernelGGL(permute_bwd_kernel<false>, grid, dim3(256), 0, s, d, pa, dxs, roa, dx,
                       (long long)max_rows);
  return hipGetLastError();
}

hipError_t launch_route_bwd(const Dims& d, const int* idx, const float* gate,
                            const float* d_gate, float* d_logits, hipStream_t s) {
  hipLaunchKernelGGL(route_bwd_kernel, dim3((d.T + 3) / 4), dim3(256), 0, s, d, idx, gate, d_gate,
                     d_logits);
  return hipGetLastError();
}

hipError_t launch_gmm_bwd(const Dims& d, const GemmBwdArgs& a, hipStream_t s) {
  const int e_res = d.S_res * d.El;
  const long long rows = a.max_rows;
  char* ws = (char*)a.scratch;
  const size_t el = d.bf16 ? 2 : 4;
  int* tile_off = (int*)ws;
  ws += a256((size_t)(d.G_res + 1) * 4);
  void* d_h = ws;
  ws += 2 * a256((size_t)rows * d.F * el);
  void* act = ws;
  ws += a256((size_t)rows * d.F * el);
  void* d_a = ws;
  if (!d.bf16) {
    F32Bwd P;
    P.x = (const float*)a.x_sorted;
    P.wg = (const float*)a.wg;
    P.wu = (const float*)a.wu;
    P.wd = (const float*)a.wd;
    P.d_out = (const float*)a.d_out;
    P.d_h = (float*)d_h;
    P.act = (float*)act;
    P.dxs = (float*)a.dx_sorted;
    P.dwg = a.dwg;
    P.dwu = a.dwu;
    P.dwd = a.dwd;
    P.group_offsets = a.group_offsets;
    P.slot_expert = a.slot_expert;
    P.G = d.G_res;
    P.H = d.H;
    P.F = d.F;
    P.lo_slot = d.lo_slot;
    P.e_base = d.e_base;
    P.e_res = e_res;
    P.max_rows = rows;
    P.accumulate = a.accumulate;
    const long long n1 = rows * d.F, n2 = rows * d.H, n3 = (long long)e_res * d.F * d.H;
    hipLaunchKernelGGL(f32_dh_kernel, dim3((unsigned)((n1 + 255) / 256)), dim3(256), 0, s, P);
    hipLaunchKernelGGL(f32_dx_kernel, dim3((unsigned)((n2 + 255) / 256)), dim3(256), 0, s, P);
    for (int which = 0; which < 3; ++which)
      hipLaunchKernelGGL(f32_dw_kernel, dim3((unsigned)((n3 + 255) / 256)), dim3(256), 0, s, P,
                         which);
    return hipGetLastError();
  }
  long long lim = (long long)d.T * d.k;
  if (rows < lim) lim = rows;
  hipLaunchKernelGGL(bwd_tiles_kernel, dim3(1), dim3(1024), 0, s, d.G_res, (int)lim,
                     a.group_offsets, tile_off);
  const long long mt_ub = (rows + kBM - 1) / kBM + d.G_res;
  DgradParams P;
  P.group_offsets = a.group_offsets;
  P.tile_off = tile_off;
  P.slot_expert = a.slot_expert;
  P.G = d.G_res;
  P.lo_slot = d.lo_slot;
  P.e_base = d.e_base;
  P.e_res = e_res;
  P.max_rows = rows;
  P.a_rows = (int)rows;
  P.d_a = nullptr;
  P.d_h = nullptr;
  P.act = nullptr;
  // d_a = d_out Wd  (K = H, against Wd^T [F, H])
  P.A = (const uint16_t*)a.d_out;
  P.B0 = P.B1 = (const uint16_t*)a.wd_t;
  P.b_stride = (size_t)d.F * d.H;
  P.C = (uint16_t*)d_a;
  P.K = d.H;
  P.Nout = d.F;
  P.n_ntiles = d.F / kBN;
  hipLaunchKernelGGL(dgrad_kernel<false>, dim3((unsigned)(mt_ub * P.n_ntiles)), dim3(256), 0, s,
                     P);
  // gate and up products recomputed; SwiGLU backward and the activation
  DgradParams Q = P;
  Q.A = (const uint16_t*)a.x_sorted;
  Q.B0 = (const uint16_t*)a.wg;
  Q.B1 = (const uint16_t*)a.wu;
  Q.C = nullptr;
  Q.d_a = (const uint16_t*)d_a;
  Q.d_h = (uint16_t*)d_h;
  Q.act = (uint16_t*)act;
  hipLaunchKernelGGL(dgrad_kernel<true>, dim3((unsigned)(mt_ub * Q.n_ntiles)), dim3(256), 0, s,
                     Q);
  // dx_sorted = [d_hg | d_hu] [Wg ; Wu]  (K = 2F, against [Wg ; Wu]^T [H, 2F])
  DgradParams X = P;
  X.A = (const uint16_t*)d_h;
  X.B0 = X.B1 = (const uint16_t*)a.wgu_t;
  X.b_stride = (size_t)d.H * 2 * d.F;
  X.C = (uint16_t*)a.dx_sorted;
  X.K = 2 * d.F;
  X.Nout = d.H;
  X.n_ntiles = d.H / kBN;
  hipLaunchKernelGGL(dgrad_kernel<false>, dim3((unsigned)(mt_ub * X.n_ntiles)), dim3(256), 0, s,
                     X);
  // [dWg ; dWu] = [d_hg | d_hu]^T x_sorted
  WgradParams W;
  W.Pm = (const uint16_t*)d_h;
  W.Qm = (const uint16_t*)a.x_sorted;
  W.C0 = a.dwg;
  W.C1 = a.dwu;
  W.c_stride = (size_t)d.F * d.H;
  W.I = 2 * d.F;
  W.J = d.H;
  W.i_split = d.F;
  W.group_offsets = a.group_offsets;
  W.slot_expert = a.slot_expert;
  W.G = d.G_res;
  W.lo_slot = d.lo_slot;
  W.e_base = d.e_base;
  W.e_res = e_res;
  W.max_rows = rows;
  W.accumulate = a.accumulate;
  W.ni_tiles = W.I / 128;
  W.nj_tiles = W.J / 128;
  hipLaunchKernelGGL(wgrad_kernel, dim3((unsigned)(e_res * W.ni_tiles * W.nj_tiles)), dim3(256),
                     0, s, W);
  // dWd = d_out^T act
  WgradParams V = W;
  V.Pm = (const uint16_t*)a.d_out;
  V.Qm = (const uint16_t*)act;
  V.C0 = V.C1 = a.dwd;
  V.I = d.H;
  V.J = d.F;
  V.i_split = d.H;
  V.ni_tiles = V.I / 128;
  V.nj_tiles = V.J / 128;
  hipLaunchKernelGGL(wgrad_kernel, dim3((unsigned)(e_res * V.ni_tiles * V.nj_tiles)), dim3(256),
                     0, s, V);
  return hipGetLastError();
}

}  // namespace moe
