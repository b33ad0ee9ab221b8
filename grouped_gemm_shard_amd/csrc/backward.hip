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
//      d_a  = d_out Wd                          (GEMM, K = H)
//      d_hg = d_a h_u SiLU'(h_g), d_hu = d_a SiLU(h_g), a = SiLU(h_g) h_u
//           (the forward's GEMM1 recomputed, SwiGLU backward in its epilogue)
//      dx_sorted = [d_hg | d_hu] [Wg ; Wu]      (GEMM, K = 2F)
//      [dWg ; dWu] = [d_hg | d_hu]^T x_sorted,  dWd = d_out^T a
//                                               (reductions over each
//                                                expert's ragged rows)
//    Where an operand is stored with the reduction index as its row (Wd
//    and Wg/Wu in the d_a and dx GEMMs, both operands of the weight
//    gradients), its rows are staged in LDS as they are and the MFMA
//    fragments are read with gfx950's LDS transpose read, so no transposed
//    copy is ever made.  With 256-row tiles (H >= 2048) d_a, dx_sorted, the
//    gate/up recompute and the layer call's expert outputs run on the
//    forward's grouped-GEMM kernel (gmm.hip: its reduction-major-B mode for
//    d_a and dx, the SwiGLU backward in its first GEMM's epilogue for the
//    recompute); the kernels here cover the other shapes;
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

// what: bit 0 writes the rows g * dy, bit 1 the gate gradients <dy, out>;
// bit 2 makes the rows dy ungated and writes each row's gate to row_gate;
// bit 3 takes the gate gradient of a row as the sum of its F/32 parts
// dg_part [r, .] (= <dy Wd, act>, the same quantity) instead of reading out.
template <bool BF16>
__global__ __launch_bounds__(256) void combine_bwd_kernel(Dims d, PassArgs pa, LayoutSet ls,
                                                          const void* dy, const void* out,
                                                          const int* roa, long long roa_stride,
                                                          const float* gate, void* d_out,
                                                          float* d_gate, long long max_rows,
                                                          int what, float* row_gate,
                                                          const float* dg_part) {
  const PassInfo pi = resolve_pass(pa);
  if (!pi.active) return;
  roa += (size_t)layout_set_of(ls, pi.j) * roa_stride;
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (i >= pass_tokens(d, pi)) return;
  const int t = pass_token(d, pi, i);
  const int lane = threadIdx.x & 63;
  constexpr int N = Vec<BF16>::N;
  const bool ungated = what & 4, parts = what & 8;
  const bool rows = what & 1, dots = (what & 2) && !parts;
  const int nparts = d.F / 32;
  for (int j = 0; j < d.k; ++j) {
    const int r = roa[(size_t)t * d.k + j];
    float dot = 0.0f;
    if (r >= 0 && r < max_rows) {
      const float g = gate[(size_t)t * d.k + j];
      if (rows && ungated && lane == 0) row_gate[r] = g;
      if (parts && (what & 2))
        for (int b = lane; b < nparts; b += 64) dot += dg_part[(size_t)r * nparts + b];
      if (rows || dots)
        for (int c = lane * N; c < d.H; c += 64 * N) {
          Vec<BF16> a;
          a.load(dy, (size_t)t * d.H + c);
          if (dots) {
            Vec<BF16> o;
            o.load(out, (size_t)r * d.H + c);
#pragma unroll
            for (int q = 0; q < N; ++q) dot = fmaf(a.v[q], o.v[q], dot);
          }
          if (rows) {
            if (!ungated) {
#pragma unroll
              for (int q = 0; q < N; ++q) a.v[q] *= g;
            }
            a.store(d_out, (size_t)r * d.H + c);
          }
        }
    }
    if (what & 2) {
      dot = wave_sum(dot);
      if (lane == 0) d_gate[(size_t)t * d.k + j] = dot;
    }
  }
}

// ---- permute backward ------------------------------------------------------

template <bool BF16>
__global__ __launch_bounds__(256) void permute_bwd_kernel(Dims d, PassArgs pa, LayoutSet ls,
                                                          const void* dxs, const int* roa,
                                                          long long roa_stride, void* dx,
                                                          long long max_rows) {
  const PassInfo pi = resolve_pass(pa);
  if (!pi.active) return;
  roa += (size_t)layout_set_of(ls, pi.j) * roa_stride;
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

// ---- m-tiles of the data-gradient GEMMs ------------------------------------

constexpr int kBM = 128;  // rows per tile
constexpr int kBN = 128;  // output columns per tile
constexpr int kBK = 32;   // reduction columns per stage
constexpr int kNST = 3;   // ring stages

// The pass's group offsets, copied to go_copy (layout pi.j of a layer
// call's passes, go_stride apart; all zero, i.e. no rows, for a pass slot
// that is not taken), and tile_off[g] = m-tiles of groups before g (kBM rows
// each).  Every later kernel of the backward reads go_copy.  Offsets that
// are not non-decreasing within [0, limit] give no tiles.
__global__ __launch_bounds__(1024) void bwd_tiles_kernel(int G, int limit, PassArgs pa,
                                                         const int* group_offsets, int go_stride,
                                                         int* go_copy, int* tile_off) {
  __shared__ int wsum[16];
  __shared__ int bad;
  if (threadIdx.x == 0) bad = 0;
  __syncthreads();
  const PassInfo pi = resolve_pass(pa);
  group_offsets += (size_t)pi.j * go_stride;
  const int g = threadIdx.x, lane = g & 63, w = g >> 6;
  for (int x = g; x <= G; x += blockDim.x) go_copy[x] = pi.active ? group_offsets[x] : 0;
  int v = 0;
  if (g < G && pi.active) {
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

// Unit of the launch this block runs, or -1.  Blocks go round-robin over
// the 8 XCDs (block b to XCD b % 8).  Each round of nb blocks (the blocks
// resident on the chip at once, a multiple of 8; the grid is whole rounds)
// covers that many consecutive units of the `total` units, and XCD x takes
// the x-th eighth of the round, so the units one XCD runs together are
// neighbours in the unit order and share their operand panels in its L2.
__device__ __forceinline__ int xcd_unit(int nb, int total) {
  const int bid = blockIdx.x;
  const int rbase = (bid / nb) * nb;
  const int rs = min(nb, total - rbase);
  if (rs <= 0) return -1;
  const int x = bid & 7, slot = (bid - rbase) >> 3;
  const int L = rbase + (x * rs >> 3) + slot;
  return L < rbase + ((x + 1) * rs >> 3) ? L : -1;
}

// 16-byte chunk permutation of a 256-byte LDS row (16 chunks): the
// transpose reads of 4 consecutive rows at one column land on disjoint
// 64-byte bank windows.
__device__ __forceinline__ int wswz(int row) { return (row & 3) << 2; }

// The same for the two-group weight-gradient loop, whose transpose reads
// take 32 bytes from each of rows 8g + k (k < 4) for the read's 16-lane
// groups g: row bit 3 also moves odd groups to the other 32-byte half of
// each 64-byte window, so a read's 512 bytes cover each of the 64 banks
// exactly twice (with bits 0-1 alone, all four groups shared 32 banks).
__device__ __forceinline__ int ppswz(int row) { return ((row & 3) << 2) | ((row >> 2) & 2); }

typedef short v4i16 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return (unsigned)(size_t)(const __attribute__((address_space(3))) char*)p;
}

// ds_read_b64_tr_b16 as inline asm: the compiler cannot tell that the
// builtin's LDS read does not alias the ring's in-flight buffer loads into
// LDS, and waits for all of them before it; here the ring's own barrier
// already guarantees the stage being read has landed.  The result is
// pending until lgkm_wait_tie.
__device__ __forceinline__ void lds_read_tr16(v4i16& r, unsigned addr) {
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(r) : "v"(addr) : "memory");
}

// Waits until at most N LDS reads of this wave are outstanding; the
// registers of one slice are tied to the wait so their uses stay after it.
template <int N>
__device__ __forceinline__ void lgkm_wait_tie(v4i16 (&a)[2][2], v4i16 (&b)[2][2]) {
  asm volatile("s_waitcnt lgkmcnt(%8)"
               : "+v"(a[0][0]), "+v"(a[0][1]), "+v"(a[1][0]), "+v"(a[1][1]), "+v"(b[0][0]),
                 "+v"(b[0][1]), "+v"(b[1][0]), "+v"(b[1][1])
               : "n"(N));
}

__device__ __forceinline__ void lgkm_wait_tie(v4i16 (&b)[2][2]) {
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(b[0][0]), "+v"(b[0][1]), "+v"(b[1][0]), "+v"(b[1][1]));
}

__device__ __forceinline__ bf16x8 join8(const v4i16& lo, const v4i16& hi) {
  bf16x8 v;
  __builtin_memcpy(&v, &lo, 8);
  __builtin_memcpy(reinterpret_cast<char*>(&v) + 8, &hi, 8);
  return v;
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
  int round_blocks;         // blocks per round (xcd_unit)
  int k_split;              // reduction-major B: rows [0, k_split) from B0, the rest from B1
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

  // units: m-tiles by n-tiles, n fastest (an XCD's run of units covers a
  // few m-tiles by all n-tiles: the A rows are read once per XCD)
  const int total = P.tile_off[P.G];
  const int unit = xcd_unit(P.round_blocks, total * P.n_ntiles);
  if (unit < 0) return;
  const int nt = unit % P.n_ntiles;
  const int m = unit / P.n_ntiles;
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

// Plain tile C = A B with B stored reduction-major, [K][Nout] per expert
// (the weights as they are: Wd [H, F] for d_a = d_out Wd, and Wg, Wu
// [F, H] stacked along K for dx = d_hg Wg + d_hu Wu), so no transposed
// copy is needed.  A stages as in dgrad_tile; B stages 32 reduction rows of
// the tile's 128 columns (256 bytes each), and its fragments come from
// ds_read_b64_tr_b16, which hands each lane 4 consecutive reduction rows of
// one column (the same reads as the weight-gradient kernel).
__device__ __forceinline__ void dgrad_kmajor_tile(const DgradParams& P) {
  constexpr int RB = kBK * 2;                  // A: 64 bytes per row per stage
  constexpr int CPR = kBK / 8;
  constexpr int RPI = 1024 / RB;
  constexpr int AI = kBM / RPI / 4;            // 2
  constexpr int BRB = kBN * 2;                 // B: 256 bytes per reduction row
  constexpr int BI = kBK * BRB / 1024 / 4;     // 2
  constexpr int LPS = AI + BI;
  constexpr int SA = kBM * RB, SS = SA + kBK * BRB;
  __shared__ __attribute__((aligned(1024))) char smem[kNST * SS];

  const int total = P.tile_off[P.G];
  const int unit = xcd_unit(P.round_blocks, total * P.n_ntiles);
  if (unit < 0) return;
  const int nt = unit % P.n_ntiles;
  const int m = unit / P.n_ntiles;
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
  const __amdgpu_buffer_rsrc_t rb0 =
      raw_rsrc(P.B0 + (size_t)e * P.b_stride, (unsigned)P.k_split * P.Nout * 2);
  const __amdgpu_buffer_rsrc_t rb1 =
      raw_rsrc(P.B1 + (size_t)e * P.b_stride, (unsigned)(K - P.k_split) * P.Nout * 2);
  int a_off[AI], b_off[BI];
#pragma unroll
  for (int i = 0; i < AI; ++i) {
    const int row = (i * 4 + w) * RPI + lane / CPR;
    a_off[i] = row < rows ? (row0 + row) * K * 2 + (((lane % CPR) ^ swz4(row)) << 4)
                          : (int)0x80000000;
  }
#pragma unroll
  for (int i = 0; i < BI; ++i) {
    const int kr = (i * 4 + w) * 4 + (lane >> 4);  // reduction row within the stage
    b_off[i] = kr * P.Nout * 2 + nt * kBN * 2 + (((lane & 15) ^ wswz(kr)) << 4);
  }
  auto issue = [&](int step) {
    char* st = smem + (step % kNST) * SS;
    const int k0 = step * kBK;
#pragma unroll
    for (int i = 0; i < AI; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(st + (i * 4 + w) * RPI * RB), 16,
                                               a_off[i], k0 * 2, 0, 0);
    // a stage's 32 reduction rows lie in one of the two stacked matrices
    const bool second = k0 >= P.k_split;
    const int kb = (second ? k0 - P.k_split : k0) * P.Nout * 2;
#pragma unroll
    for (int i = 0; i < BI; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(second ? rb1 : rb0,
                                               (lds_void*)(st + SA + (i * 4 + w) * 1024), 16,
                                               b_off[i], kb, 0, 0);
  };

  floatx16 acc[2][2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[mi][ni][q] = 0.0f;
  int a_row[2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) a_row[mi] = wm * 64 + mi * 32 + (lane & 31);
  // transpose-read offsets of B (see wgrad_tile)
  const int G4 = lane >> 4, s4 = lane & 15;
  const int trow = 8 * (G4 >> 1) + (s4 >> 2);
  const int tcol = 16 * (G4 & 1) + 4 * (s4 & 3);
  unsigned b_tr[2];
#pragma unroll
  for (int ni = 0; ni < 2; ++ni) {
    const int c = wn * 64 + ni * 32 + tcol;
    b_tr[ni] = SA + trow * BRB + (((c >> 3) ^ wswz(trow)) << 4) + (c & 7) * 2;
  }
  const unsigned lds0 = lds_addr(smem);

#pragma unroll
  for (int s0 = 0; s0 < kNST - 1; ++s0)
    if (s0 < KT) issue(s0);
  for (int kt = 0; kt < KT; ++kt) {
    if (kt + 1 < KT) wait_vm_barrier<LPS>();
    else wait_vm_barrier<0>();
    if (kt + kNST - 1 < KT) issue(kt + kNST - 1);
    const char* sa = smem + (kt % kNST) * SS;
    const unsigned st = lds0 + (kt % kNST) * SS;
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      v4i16 rb[2][2];
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          lds_read_tr16(rb[ni][h], st + b_tr[ni] + (ks * 16 + 4 * h) * BRB);
      const int kc = ks * 2 + (lane >> 5);
      bf16x8 a[2];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
        a[mi] = *(const bf16x8*)(sa + a_row[mi] * RB + ((kc ^ swz4(a_row[mi])) << 4));
      lgkm_wait_tie(rb);
      bf16x8 b[2];
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) b[ni] = join8(rb[ni][0], rb[ni][1]);
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mi], b[ni], acc[mi][ni], 0, 0, 0);
    }
  }

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
        P.C[r * P.Nout + c] = f2bf(acc[mi][ni][q]);
      }
    }
}

__global__ __launch_bounds__(256, 2) void dgrad_kmajor_kernel(DgradParams P) {
  dgrad_kmajor_tile(P);
}

// ---- weight-gradient GEMM --------------------------------------------------
//
// dW[e] = P^T Q summed over the rows of every group of expert e (P, Q
// row-major with the row as the reduction index).  The rows of an expert
// are cut into chunks of at most Kc rows (Kc sized so that the longest
// chunk is no more than the chip's average share of the launch), so a hot
// expert's reduction runs on several workgroups; an expert with one chunk
// writes its gradient directly, the chunks of a split expert write float32
// partials that a second kernel adds in chunk order (deterministic).

constexpr int kWBK = 32;   // rows per stage
constexpr int kWNST = 4;   // ring stages
constexpr int kWMaxRes = 1024;
constexpr int kWMaxChunks = 2048;
constexpr int kWOld = 16;  // 16-byte runs per thread of a 128 x 128 float tile

// Per-expert plan of the weight-gradient launches, from the group offsets:
// the expert's groups in group order (their first row and row count, as a
// list per expert), its rows R_e, its chunk count nch_e = max(1,
// ceil(R_e / Kc)), the first chunk index, and for split experts the first
// partial slot.  chunk_e / chunk_i map a chunk to (expert, index); unused
// chunk slots hold -1.  Offsets that are not non-decreasing within
// [0, max_rows] count as empty groups.
struct WgradPlan {
  int* grp_off;    // [e_res + 1]
  int* grp_row0;   // [G]
  int* grp_len;    // [G]
  int* rows;       // [e_res]
  int* nch;        // [e_res]
  int* pbase;      // [e_res]
  int* chunk_e;    // [nc_ub]
  int* chunk_i;    // [nc_ub]
  int* order_e;    // [nc_ub] chunks by row count, longest first (ties: chunk order)
  int* order_i;    // [nc_ub]
  int* meta;       // [0] chunks in use
};

// The groups are `nsets` sets of G (the passes of a layer call whose weight
// gradients are taken together): set s's offsets are group_offsets[s (G+1)
// ...] over rows s * row_stride + [0, max_rows) of the operands.  A set
// with malformed offsets leaves every group empty.
__global__ __launch_bounds__(1024) void wgrad_plan_kernel(WgradPlan W, const int* group_offsets,
                                                          const int* slot_expert, int G,
                                                          int nsets, long long row_stride,
                                                          int lo_slot, int e_base, int e_res,
                                                          long long max_rows, int kc, int nc_ub) {
  __shared__ int ge[kMaxSlots], gr[kMaxSlots], g0[kMaxSlots];
  __shared__ int gcnt[kWMaxRes], rsum[kWMaxRes], cb[kWMaxRes + 1];
  __shared__ int bad;
  const int tid = threadIdx.x;
  if (tid == 0) bad = 0;
  __syncthreads();
  const int Gs = G;
  G = nsets * Gs;  // <= kMaxSlots (host)
  for (int g = tid; g < G; g += blockDim.x) {
    const int set = g / Gs, gg = g - set * Gs;
    const int* go = group_offsets + (size_t)set * (Gs + 1);
    const int a = go[gg], b = go[gg + 1];
    if (a < 0 || b < a || b > max_rows) bad = 1;
    const int e = slot_expert[lo_slot + gg] - e_base;
    ge[g] = (e >= 0 && e < e_res) ? e : -1;
    gr[g] = b - a;
    g0[g] = (int)(set * row_stride) + a;
  }
  __syncthreads();
  // a malformed offset sequence leaves every group empty, so the rows of
  // all experts together never exceed max_rows (which bounds the chunks
  // and partial slots)
  if (bad)
    for (int g = tid; g < G; g += blockDim.x) ge[g] = -1;
  __syncthreads();
  for (int e = tid; e < e_res; e += blockDim.x) {
    int c = 0, r = 0;
    for (int g = 0; g < G; ++g)
      if (ge[g] == e) {
        ++c;
        r += gr[g];
      }
    gcnt[e] = c;
    rsum[e] = r;
  }
  __syncthreads();
  if (tid == 0) {
    int go = 0, co = 0, po = 0;
    for (int e = 0; e < e_res; ++e) {
      W.grp_off[e] = go;
      go += gcnt[e];
      const int n = rsum[e] > kc ? (rsum[e] + kc - 1) / kc : 1;
      W.rows[e] = rsum[e];
      W.nch[e] = n;
      W.pbase[e] = n > 1 ? po : -1;
      if (n > 1) po += n;
      cb[e] = co;
      co += n;
    }
    W.grp_off[e_res] = go;
    cb[e_res] = co;
    W.meta[0] = min(min(co, nc_ub), kWMaxChunks);
  }
  __syncthreads();
  for (int e = tid; e < e_res; e += blockDim.x) {
    int o = W.grp_off[e];
    for (int g = 0; g < G; ++g)
      if (ge[g] == e) {
        W.grp_row0[o] = g0[g];
        W.grp_len[o] = gr[g];
        ++o;
      }
    for (int c = cb[e]; c < cb[e + 1] && c < nc_ub; ++c) {
      W.chunk_e[c] = e;
      W.chunk_i[c] = c - cb[e];
    }
  }
  for (int c = cb[e_res] + tid; c < nc_ub; c += blockDim.x) {
    W.chunk_e[c] = -1;
    W.chunk_i[c] = 0;
  }
  __syncthreads();
  // chunks by row count, longest first: a round of the launch then holds
  // chunks of about the same length on every XCD
  // (at most e_res + max_rows / kc <= 1024 + 256 chunks: kc >= max_rows/256)
  __shared__ int len_s[kWMaxChunks];
  const int nc = min(min(cb[e_res], nc_ub), kWMaxChunks);
  for (int c = tid; c < nc; c += blockDim.x)
    len_s[c] = min(kc, rsum[W.chunk_e[c]] - W.chunk_i[c] * kc);
  __syncthreads();
  for (int c = tid; c < nc; c += blockDim.x) {
    const int lc = len_s[c];
    int rank = 0;
    for (int o = 0; o < nc; ++o) {
      const int lo = len_s[o];
      rank += (lo > lc || (lo == lc && o < c)) ? 1 : 0;
    }
    W.order_e[rank] = W.chunk_e[c];
    W.order_i[rank] = W.chunk_i[c];
  }
}

struct WgradParams {
  const uint16_t* Pm;   // [a_rows, I] (row-major, I contiguous)
  const uint16_t* Qm;   // [a_rows, J]
  float* C0;            // rows i < i_split: C0[e][i][j]
  float* C1;            // rows i >= i_split: C1[e][i - i_split][j]
  float* part;          // [slots][I][J] partials of split experts
  size_t c_stride;      // elements per expert of C0 / C1
  int I, J, i_split;
  int a_rows;
  WgradPlan plan;
  int kc, ni_tiles, nj_tiles;
  long long slots;      // partial slots in part
  int accumulate;
  int round_blocks;     // 256 x 256 tiles: blocks per round (xcd_unit)
};

constexpr int kWMaxGroups = 1024;  // groups of one expert kept in LDS

// Actual row of position p of the expert's row sequence, from the LDS copy
// of its group list (first rows, then lengths); cur is the lane's group
// cursor (positions only grow), base the sequence start of group cur.  No
// global loads: the ring's loads stay the only vector-memory operations in
// flight, so waiting for one stage never waits for a later one.
__device__ __forceinline__ int wgrad_row(const int* gl, int ng, int p, int& cur, int& base) {
  while (cur < ng && p >= base + gl[kWMaxGroups + cur]) {
    base += gl[kWMaxGroups + cur];
    ++cur;
  }
  return cur < ng ? gl[cur] + (p - base) : -1;
}


// The 4 MFMAs of one 16-row slice (2 x 2 tiles of 32 x 32).
__device__ __forceinline__ void mma_slice(const v4i16 (&a)[2][2], const v4i16 (&b)[2][2],
                                          floatx16 (&acc)[2][2]) {
  bf16x8 fa[2], fb[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    fa[m] = join8(a[m][0], a[m][1]);
    fb[m] = join8(b[m][0], b[m][1]);
  }
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
      acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[mi], fb[ni], acc[mi][ni], 0, 0, 0);
}

// One 128 x 128 tile of one chunk.  4 waves in a 2 x 2 grid, 64 x 64 per
// wave.  Raw rows of both operands (256 bytes of the tile's columns each)
// go from HBM into a 4-stage LDS ring with buffer_load ... lds; the MFMA
// fragments are read with ds_read_tr16_b64, which hands each lane 4
// consecutive rows of one column: lane 4a+b of each 16-lane group receives
// element b of the 8-byte runs that lanes a, a+4, a+8 and a+12 address.
__device__ __forceinline__ void wgrad_tile(const WgradParams& P, char* smem, int* gl) {
  constexpr int RB = 256;                 // bytes per staged row (128 columns)
  constexpr int OPB = kWBK * RB;          // one operand's stage (8 KB)
  constexpr int SS = 2 * OPB;             // stage
  constexpr int LPO = OPB / 1024 / 4;     // loads per wave per operand per stage (2)
  constexpr int LPS = 2 * LPO;
  const int tiles = P.ni_tiles * P.nj_tiles;
  // units: chunks (longest first) by tiles, tiles fastest, in block order.
  // Consecutive blocks go to different XCDs, so each XCD runs a share of
  // every chunk's tiles.  (Running whole chunks per XCD fetches every row
  // from HBM once instead of ~4.5 times, but measured 15% slower: an XCD's
  // workgroups then all read the same rows at once.)
  const int u = blockIdx.x / tiles;
  const int t = blockIdx.x % tiles;
  if (u >= P.plan.meta[0]) return;
  const int e = P.plan.order_e[u];
  if (e < 0) return;
  const int ci = P.plan.order_i[u];
  const int it = t / P.nj_tiles, jt = t % P.nj_tiles;
  const int i0 = it * 128, j0 = jt * 128;
  const int R = P.plan.rows[e], nch = P.plan.nch[e];
  const int k0 = ci * P.kc, k1 = min(R, k0 + P.kc);
  const int KT = k1 > k0 ? (k1 - k0 + kWBK - 1) / kWBK : 0;
  const int g_lo = P.plan.grp_off[e];
  const int ng = min(P.plan.grp_off[e + 1] - g_lo, kWMaxGroups);
  const bool direct = nch == 1;
  const long long slot = direct ? 0 : (long long)P.plan.pbase[e] + ci;
  if (!direct && (P.plan.pbase[e] < 0 || slot >= P.slots)) return;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int x = tid; x < ng; x += blockDim.x) {
    gl[x] = P.plan.grp_row0[g_lo + x];
    gl[kWMaxGroups + x] = P.plan.grp_len[g_lo + x];
  }
  __syncthreads();
  const int wm = w >> 1, wn = w & 1;
  const __amdgpu_buffer_rsrc_t rp = raw_rsrc(P.Pm, (unsigned)P.a_rows * P.I * 2);
  const __amdgpu_buffer_rsrc_t rq = raw_rsrc(P.Qm, (unsigned)P.a_rows * P.J * 2);
  // this lane's staged rows (one per load) and their group cursors
  int cur[LPO], base[LPO];
#pragma unroll
  for (int i = 0; i < LPO; ++i) {
    cur[i] = 0;
    base[i] = 0;
  }
  const int pch = lane & 15;  // physical 16-byte chunk of the lane's load
  auto issue = [&](int step) {
    char* st = smem + (step % kWNST) * SS;
#pragma unroll
    for (int i = 0; i < LPO; ++i) {
      const int rr = (i * 4 + w) * 4 + (lane >> 4);  // row within the stage
      const int p = k0 + step * kWBK + rr;
      const int row = p < k1 ? wgrad_row(gl, ng, p, cur[i], base[i]) : -1;
      const int lch = pch ^ wswz(rr);
      const int po = row >= 0 ? row * P.I * 2 + i0 * 2 + lch * 16 : (int)0x80000000;
      const int qo = row >= 0 ? row * P.J * 2 + j0 * 2 + lch * 16 : (int)0x80000000;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rp, (lds_void*)(st + (i * 4 + w) * 1024), 16, po,
                                               0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (lds_void*)(st + OPB + (i * 4 + w) * 1024), 16,
                                               qo, 0, 0, 0);
    }
  };

  floatx16 acc[2][2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[mi][ni][q] = 0.0f;

  // transpose-read addressing: source lane (group G = lane/16, s = lane%16)
  // points at row 8*(G/2) + s/4 (+4 for the second half of the 8 values)
  // and column 16*(G%2) + 4*(s%4) of the wave's 32-column MFMA tile.  The
  // row's chunk permutation depends only on row % 4 = s/4, so each lane's
  // reads differ by whole rows (constant byte offsets).
  const int G = lane >> 4, s = lane & 15;
  const int trow = 8 * (G >> 1) + (s >> 2);
  const int tcol = 16 * (G & 1) + 4 * (s & 3);
  unsigned a_off[2], b_off[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int ca = wm * 64 + m * 32 + tcol, cb = wn * 64 + m * 32 + tcol;
    a_off[m] = trow * RB + (((ca >> 3) ^ wswz(trow)) << 4) + (ca & 7) * 2;
    b_off[m] = OPB + trow * RB + (((cb >> 3) ^ wswz(trow)) << 4) + (cb & 7) * 2;
  }
  const unsigned lds0 = lds_addr(smem);

  if (direct && P.accumulate && KT == 0) return;
  float* part = direct ? nullptr : P.part + (size_t)slot * P.I * P.J;
  // element (i, j) of expert e's gradient, or of the chunk's partial
  auto out_ptr = [&](int i, int j) {
    if (!direct) return part + (size_t)i * P.J + j;
    if (i < P.i_split) return P.C0 + (size_t)e * P.c_stride + (size_t)i * P.J + j;
    return P.C1 + (size_t)e * P.c_stride + (size_t)(i - P.i_split) * P.J + j;
  };
  // an accumulated gradient's old values, 16-byte runs of the tile's rows
  // (thread tid: rows tid/32 + 8m, columns 4 (tid%32) ...), loaded now so
  // that their latency passes during the reduction loop
  const bool rmw = direct && P.accumulate;
  float4 old[kWOld];
  if (rmw) {
#pragma unroll
    for (int m = 0; m < kWOld; ++m)
      old[m] = *(const float4*)out_ptr(i0 + (tid >> 5) + 8 * m, j0 + (tid & 31) * 4);
  }

#pragma unroll
  for (int s0 = 0; s0 < kWNST - 1; ++s0)
    if (s0 < KT) issue(s0);
  for (int kt = 0; kt < KT; ++kt) {
    const int ahead = min(KT - 1 - kt, kWNST - 2);
    if (ahead >= 2) wait_vm_barrier<2 * LPS>();
    else if (ahead == 1) wait_vm_barrier<LPS>();
    else wait_vm_barrier<0>();
    if (kt + kWNST - 1 < KT) issue(kt + kWNST - 1);
    const unsigned st = lds0 + (kt % kWNST) * SS;
    // both 16-row slices' fragments: [slice][mi or ni][half]
    v4i16 ra[2][2][2], rb[2][2][2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const unsigned dr = (ks * 16 + 4 * h) * RB;
          lds_read_tr16(ra[ks][m][h], st + a_off[m] + dr);
          lds_read_tr16(rb[ks][m][h], st + b_off[m] + dr);
        }
    lgkm_wait_tie<8>(ra[0], rb[0]);
    mma_slice(ra[0], rb[0], acc);
    lgkm_wait_tie<0>(ra[1], rb[1]);
    mma_slice(ra[1], rb[1], acc);
  }

  // a single-chunk expert writes its gradient (skipped when there is
  // nothing to add), a split expert's chunk its partial.  The tile goes
  // through LDS (the ring, 64 KB = 128 x 128 floats) so that every thread
  // then reads, adds and stores whole 16-byte runs of rows; the old values
  // of an accumulated gradient were loaded before the reduction loop.
  __syncthreads();  // every wave is done with the ring
  float* tile = (float*)smem;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int i = wm * 64 + mi * 32 + (q >> 2) * 8 + (lane >> 5) * 4 + (q & 3);
        const int j = wn * 64 + ni * 32 + (lane & 31);
        tile[i * 128 + j] = acc[mi][ni][q];
      }
  __syncthreads();
#pragma unroll
  for (int m = 0; m < kWOld; ++m) {
    const int i = (tid >> 5) + 8 * m, j = (tid & 31) * 4;
    float4 v = *(const float4*)(tile + i * 128 + j);
    if (rmw) {
      v.x += old[m].x;
      v.y += old[m].y;
      v.z += old[m].z;
      v.w += old[m].w;
    }
    *(float4*)out_ptr(i0 + i, j0 + j) = v;
  }
}

__global__ __launch_bounds__(256, 2) void wgrad_kernel(WgradParams P) {
  static_assert(kWNST * 2 * kWBK * 256 >= 128 * 128 * 4, "the epilogue's tile fits the ring");
  __shared__ __attribute__((aligned(1024))) char smem[kWNST * 2 * kWBK * 256];
  __shared__ int gl[2 * kWMaxGroups];
  wgrad_tile(P, smem, gl);
}

// ---- weight gradients on 256 x 256 tiles (long reductions, H >= 2048) ----
//
// The forward's two-group loop with both operands reduction-major: 8 waves
// in two groups of four (one wave of each per SIMD) take turns reading
// fragments and multiplying.  A K step is 64 reduction rows; its operands
// are four 16 KB quarters in a ring of ten (the whole LDS): P columns i0 ..
// i0+127 (read by group 0), i0+128 .. i0+255 (group 1), Q columns j0 ..
// j0+127 and j0+128 .. j0+255 (both groups).  Each quarter holds the step's
// 64 rows of its 128 columns (256-byte rows, 16-byte chunks permuted by
// row), and every MFMA fragment comes from two LDS transpose reads.  The
// issue and wait schedule is the forward's: group 0 issues quarters 4j+7 and
// 4j+8 in its read phase of step j, group 1 quarters 4j+9 and 4j+10.
//
// The rows of a step are gathered: reduction position p of the chunk is
// row grp_row0[g] + (p - start of g) of the expert's groups in order.  Each
// wave keeps a window of up to 64 groups in registers (lane l: group wb+l,
// its first row, first position and length) and walks it with uniform
// reads of single lanes, so issuing a step's loads waits on no memory
// access; the window is refilled (rarely: more than 64 groups) by plain
// loads, which only make the ring's later waits stronger, since vector
// memory loads complete in issue order.
#ifndef MOE_WGRAD_BAND
#define MOE_WGRAD_BAND 4
#endif
constexpr int kWpQ = 16384;         // bytes per quarter
constexpr int kWpRing = 10 * kWpQ;  // the whole LDS
constexpr int kWpStride = 256 + 16;  // floats per row of the epilogue's half tile

template <int OFF>
__device__ __forceinline__ void lds_tr(v4i16& r, unsigned addr) {
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF) : "memory");
}

// Waits for every LDS read of the wave, with 16 fragment registers tied to
// the wait so that no use of them is placed before it.
__device__ __forceinline__ void tie16(v4i16* r) {
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]), "+v"(r[4]), "+v"(r[5]),
                 "+v"(r[6]), "+v"(r[7]), "+v"(r[8]), "+v"(r[9]), "+v"(r[10]), "+v"(r[11]),
                 "+v"(r[12]), "+v"(r[13]), "+v"(r[14]), "+v"(r[15]));
}

template <int N>
__device__ __forceinline__ void vm_wait_n() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void lgkm_wait_all() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Workgroup barrier that no instruction is scheduled across.
__device__ __forceinline__ void phase_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ void wgrad_tile_pp(const WgradParams& P, char* smem) {
  constexpr int BK = 64, LQ = 4, NQ_PRO = 8, MI = 4, NI = 8;
  const int tiles = P.ni_tiles * P.nj_tiles;
  const int L = xcd_unit(P.round_blocks, P.plan.meta[0] * tiles);
  if (L < 0) return;
  const int u = L / tiles, t = L - u * tiles;
  const int e = P.plan.order_e[u];
  if (e < 0) return;
  const int ci = P.plan.order_i[u];
  // a chunk's tiles go in bands of up to WB tile rows, column by column:
  // the 32 tiles an XCD runs together then share a few row panels of P and
  // a few column panels of Q in its L2
  constexpr int WB = MOE_WGRAD_BAND;
  const int band = t / (WB * P.nj_tiles);
  const int bh = min(WB, P.ni_tiles - band * WB);
  const int tr = t - band * WB * P.nj_tiles;
  const int jt = tr / bh, it = band * WB + (tr - jt * bh);
  const int i0 = it * 256, j0 = jt * 256;
  const int R = P.plan.rows[e], nch = P.plan.nch[e];
  const int k0 = ci * P.kc, k1 = min(R, k0 + P.kc);
  const int KT = k1 > k0 ? (k1 - k0 + BK - 1) / BK : 0;
  const int NQ = 4 * KT;
  const int g_lo = P.plan.grp_off[e];
  const int ng = P.plan.grp_off[e + 1] - g_lo;
  const bool direct = nch == 1;
  const long long slot = direct ? 0 : (long long)P.plan.pbase[e] + ci;
  if (!direct && (P.plan.pbase[e] < 0 || slot >= P.slots)) return;
  if (direct && P.accumulate && KT == 0) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = w >> 2, wig = w & 3;
  const int wml = wig >> 1, wn = wig & 1;
  const __amdgpu_buffer_rsrc_t rp = raw_rsrc(P.Pm, (unsigned)P.a_rows * P.I * 2);
  const __amdgpu_buffer_rsrc_t rq = raw_rsrc(P.Qm, (unsigned)P.a_rows * P.J * 2);

  // the group window: lane l holds group wb + l as the end of its positions
  // and its first row minus its first position (lanes past the expert's
  // groups: length 0)
  int wb = 0, cseg = 0, cpos = 0;  // cpos: first position of group cseg
  int s_end = 0, s_rbase = 0;
  auto load_window = [&](int base, int base_pos) {
    wb = base;
    const int c = base + lane;
    const int ln = c < ng ? P.plan.grp_len[g_lo + c] : 0;
    const int r0 = c < ng ? P.plan.grp_row0[g_lo + c] : 0;
    int x = ln;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    s_end = base_pos + x;
    s_rbase = r0 - (s_end - ln);
  };
  load_window(0, 0);
  // rows of the chunk's step s for this lane's LQ loads (-1: past the
  // chunk); steps are asked for in nondecreasing order.  Load i of the lane
  // covers position 16 i + rr0 of the step.
  const int rr0 = 4 * wig + (lane >> 4);
  auto rows_of = [&](int s, int (&row)[LQ]) {
#pragma unroll
    for (int i = 0; i < LQ; ++i) row[i] = -1;
    const int lo = k0 + s * BK, hi = min(lo + BK, k1);
    // a walk past the window left group cseg behind: refill from it
    if (cseg < wb) load_window(cseg, cpos);
    // first group that ends after lo
    while (cseg < ng) {
      const int en = __builtin_amdgcn_readlane(s_end, cseg - wb);
      if (en > lo) break;
      ++cseg;
      cpos = en;
      if (cseg - wb == 64 && cseg < ng) load_window(cseg, en);
    }
    int c = cseg;
    while (c < ng) {
      if (c - wb == 64) load_window(c, __builtin_amdgcn_readlane(s_end, 63));
      const int l = c - wb;
      const int en = __builtin_amdgcn_readlane(s_end, l);
      const int rb = __builtin_amdgcn_readlane(s_rbase, l);
#pragma unroll
      for (int i = 0; i < LQ; ++i) {
        const int p = lo + 16 * i + rr0;
        if (row[i] < 0 && p < en && p < hi) row[i] = rb + p;
      }
      if (en >= hi) break;
      ++c;
    }
  };
  // quarter q = 4 step + part: P columns (parts 0, 1) or Q columns (2, 3)
  const int pch = lane & 15;
  auto issue_q = [&](int q, const int (&row)[LQ]) {
    if (q >= NQ) return;
    char* st = smem + (q % 10) * kWpQ;
    const int part = q & 3;
    const bool isp = part < 2;
    const int rowb = (isp ? P.I : P.J) * 2;
    const int colb = (isp ? i0 : j0) * 2 + (part & 1) * 256;
#pragma unroll
    for (int i = 0; i < LQ; ++i) {
      const int off = row[i] >= 0 ? row[i] * rowb + colb + ((pch ^ ppswz(rr0)) << 4)
                                  : (int)0x80000000;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(isp ? rp : rq,
                                               (lds_void*)(st + (i * 4 + wig) * 1024), 16, off,
                                               0, 0, 0);
    }
  };
  // fragment reads: lane j of 16-lane group g addresses row 8g + j/4 (+4 for
  // the second read) and columns 4 (j%4) .. of its 16-column tile
  const int tj = lane & 15;
  const unsigned tk_base =
      (8 * (lane >> 4) + (tj >> 2)) * 256 + (tj & 1) * 8 + (((tj & 3) >> 1) << 4);
  const int tk_sw = ((tj >> 2) << 2) | (((lane >> 4) & 1) << 1);  // ppswz of the lane's rows
  const unsigned lds0 = lds_addr(smem);

  floatx4 acc[MI][NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[mi][ni][q] = 0.0f;

  // prologue: steps 0 and 1 (group 0 its P quarters and Q columns 0-127,
  // group 1 its P quarters and Q columns 128-255)
  int rows[LQ];
  rows_of(0, rows);
  issue_q(grp, rows);
  issue_q(2 + grp, rows);
  if (KT > 1) {
    rows_of(1, rows);
    issue_q(4 + grp, rows);
    issue_q(6 + grp, rows);
  }
  vm_wait_n<0>();
  phase_barrier();
  if (grp == 1) phase_barrier();
  v4i16 at[2][MI][2], bt[2][NI][2];
  for (int kt = 0; kt < KT; ++kt) {
    const unsigned sa = lds0 + ((4 * kt + grp) % 10) * kWpQ + tk_base;
    const unsigned sb = lds0 + ((4 * kt + 2 + wn) % 10) * kWpQ + tk_base;
    // read phase: this group's two quarters (group 0: Q columns 128-255 of
    // step kt+1 and its P quarter of step kt+2; group 1: its P quarter and
    // Q columns 0-127 of step kt+2), then the step's fragments
    const int q0 = 4 * kt + 7 + 2 * grp, q1 = q0 + 1;
    if (grp == 0) {
      if (q0 >= NQ_PRO && q0 < NQ) {
        rows_of(kt + 1, rows);
        issue_q(q0, rows);
      }
      if (q1 < NQ) {
        rows_of(kt + 2, rows);
        issue_q(q1, rows);
      }
    } else if (q0 < NQ) {
      rows_of(kt + 2, rows);
      issue_q(q0, rows);
      issue_q(q1, rows);
    }
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      const unsigned ad = sa + (((2 * (4 * wml + mi)) ^ tk_sw) << 4);
      lds_tr<0>(at[0][mi][0], ad);
      lds_tr<1024>(at[0][mi][1], ad);
      lds_tr<8192>(at[1][mi][0], ad);
      lds_tr<9216>(at[1][mi][1], ad);
    }
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      const unsigned ad = sb + (((2 * ni) ^ tk_sw) << 4);
      lds_tr<0>(bt[0][ni][0], ad);
      lds_tr<1024>(bt[0][ni][1], ad);
      lds_tr<8192>(bt[1][ni][0], ad);
      lds_tr<9216>(bt[1][ni][1], ad);
    }
    tie16(&at[0][0][0]);
    tie16(&bt[0][0][0]);
    tie16(&bt[1][0][0]);
    if (grp == 1) {
      // quarters up to 4kt+6 landed; its two newest may stay in flight
      if (q1 < NQ) vm_wait_n<2 * LQ>();
      else if (q0 < NQ) vm_wait_n<LQ>();
      else vm_wait_n<0>();
    }
    lgkm_wait_all();
    phase_barrier();
    // multiply phase
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        const bf16x8 av = join8(at[ks][mi][0], at[ks][mi][1]);
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              av, join8(bt[ks][ni][0], bt[ks][ni][1]), acc[mi][ni], 0, 0, 0);
      }
    if (grp == 0) {
      // quarters up to 4kt+7 landed; its newest (4kt+8) may stay in flight
      if (q1 >= NQ_PRO && q1 < NQ) vm_wait_n<LQ>();
      else vm_wait_n<0>();
    }
    phase_barrier();
  }
  if (grp == 0) phase_barrier();

  // Epilogue: the tile leaves through LDS in two halves of 128 rows (group
  // h's), each thread then reading, adding and storing 16-byte runs of
  // rows.  A single-chunk expert writes its gradient (adding the old values
  // when accumulating), a split expert's chunk its partial.
  float* part = direct ? nullptr : P.part + (size_t)slot * P.I * P.J;
  auto out_ptr = [&](int i, int j) {
    if (!direct) return part + (size_t)i * P.J + j;
    if (i < P.i_split) return P.C0 + (size_t)e * P.c_stride + (size_t)i * P.J + j;
    return P.C1 + (size_t)e * P.c_stride + (size_t)(i - P.i_split) * P.J + j;
  };
  const bool rmw = direct && P.accumulate;
  float* tile = (float*)smem;
  __syncthreads();
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    if (grp == h) {
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = wml * 64 + mi * 16 + (lane >> 4) * 4 + q;
#pragma unroll
          for (int ni = 0; ni < NI; ++ni)
            tile[r * kWpStride + wn * 128 + ni * 16 + (lane & 15)] = acc[mi][ni][q];
        }
    }
    __syncthreads();
    float4 old[16];
    if (rmw) {
#pragma unroll
      for (int m = 0; m < 16; ++m)
        old[m] = *(const float4*)out_ptr(i0 + h * 128 + m * 8 + (tid >> 6), j0 + (tid & 63) * 4);
    }
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      const int r = m * 8 + (tid >> 6), c = (tid & 63) * 4;
      float4 v = *(const float4*)(tile + r * kWpStride + c);
      if (rmw) {
        v.x += old[m].x;
        v.y += old[m].y;
        v.z += old[m].z;
        v.w += old[m].w;
      }
      *(float4*)out_ptr(i0 + h * 128 + r, j0 + c) = v;
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(512, 1) void wgrad_pp_kernel(WgradParams P) {
  static_assert(128 * kWpStride * 4 <= kWpRing, "the epilogue's half tile fits the ring");
  __shared__ __attribute__((aligned(1024))) char smem[kWpRing];
  wgrad_tile_pp(P, smem);
}

// dW[e] (+)= the sum of a split expert's partials, in chunk order.
__global__ __launch_bounds__(256) void wgrad_reduce_kernel(WgradParams P) {
  const int e = blockIdx.y;
  const int n = P.plan.nch[e];
  if (n <= 1 || P.plan.pbase[e] < 0 || (long long)P.plan.pbase[e] + n > P.slots) return;
  const long long IJ = (long long)P.I * P.J;
  const long long idx = ((long long)blockIdx.x * 256 + threadIdx.x) * 4;
  if (idx >= IJ) return;
  const float* part = P.part + (size_t)P.plan.pbase[e] * IJ + idx;
  float4 s = *(const float4*)part;
  for (int c = 1; c < n; ++c) {
    const float4 v = *(const float4*)(part + (size_t)c * IJ);
    s.x += v.x;
    s.y += v.y;
    s.z += v.z;
    s.w += v.w;
  }
  const int i = (int)(idx / P.J), j = (int)(idx % P.J);
  float* dst = i < P.i_split ? P.C0 + (size_t)e * P.c_stride + (size_t)i * P.J + j
                             : P.C1 + (size_t)e * P.c_stride + (size_t)(i - P.i_split) * P.J + j;
  if (P.accumulate) {
    const float4 o = *(const float4*)dst;
    s.x += o.x;
    s.y += o.y;
    s.z += o.z;
    s.w += o.w;
  }
  *(float4*)dst = s;
}

// Rows per chunk: no chunk longer than the chip's average share of the
// launch with the fewest tiles per expert when the launch is spread over
// MOE_WGRAD_TILES workgroup slots, and at least 256.  Split experts need at
// most floor(2 max_rows / Kc) partials.  (Measured on the mid-sized layer's
// backward, 16384 rows: 256 slots, i.e. chunks of 2048 rows, beat 64, 128,
// 512, 1024 and 2048 slots by 3-30%: fewer partial gradients to write and add.)
// Weight gradients of long reductions on the 256 x 256 two-group loop (1)
// or on 128 x 128 tiles (0).
#ifndef MOE_WGRAD_PP
#define MOE_WGRAD_PP 1
#endif
#ifndef MOE_WGRAD_TILES
#define MOE_WGRAD_TILES 256
#endif
inline int wgrad_kc(const Dims& d, int64_t max_rows) {
  const long long tmin = (long long)(d.H / 128) * (d.F / 128);
  long long kc = (max_rows * tmin + MOE_WGRAD_TILES - 1) / MOE_WGRAD_TILES;
  kc = (kc + kWBK - 1) / kWBK * kWBK;
  return (int)(kc < 256 ? 256 : kc > (1 << 30) ? (1 << 30) : kc);
}
inline long long wgrad_slots(int64_t max_rows, int kc) { return 2 * max_rows / kc; }
inline long long wgrad_nc_ub(const Dims& d, int64_t max_rows, int kc) {
  return (long long)d.S_res * d.El + max_rows / kc;
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

// Blocks of one round of a kernel's unit order (xcd_unit): the compute
// units rounded down to a multiple of 8 (the XCDs) times the workgroups of
// the kernel that fit on one, cached per device and kernel.
int bwd_round_blocks(const void* kernel, int threads, int which) {
  static int cache[64][8] = {};
  static std::mutex mu;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if (cache[dev][which] == 0) {
    int cus = 0, occ = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus < 8)
      cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, threads, 0) != hipSuccess ||
        occ < 1)
      occ = 1;
    cache[dev][which] = cus / 8 * 8 * occ;
  }
  return cache[dev][which];
}

inline unsigned whole_rounds(long long units, int nb) {
  return (unsigned)((units + nb - 1) / nb * nb);
}

}  // namespace

namespace {

// Scratch of the bf16 backward after the tile offsets and the d_h, act and
// d_a rows: the weight-gradient plan and the partials of split experts.
struct WgradScratch {
  WgradPlan plan;
  float* part;
  size_t bytes;
};

WgradScratch carve_wgrad(const Dims& d, int64_t max_rows, int groups, char* base) {
  const int e_res = d.S_res * d.El;
  const int kc = wgrad_kc(d, max_rows);
  const long long nc = wgrad_nc_ub(d, max_rows, kc);
  const long long slots = wgrad_slots(max_rows, kc);
  WgradScratch w;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    char* p = base ? base + o : nullptr;
    o += a256(bytes);
    return p;
  };
  w.plan.grp_off = (int*)take((size_t)(e_res + 1) * 4);
  w.plan.grp_row0 = (int*)take((size_t)groups * 4);
  w.plan.grp_len = (int*)take((size_t)groups * 4);
  w.plan.rows = (int*)take((size_t)e_res * 4);
  w.plan.nch = (int*)take((size_t)e_res * 4);
  w.plan.pbase = (int*)take((size_t)e_res * 4);
  w.plan.chunk_e = (int*)take((size_t)nc * 4);
  w.plan.chunk_i = (int*)take((size_t)nc * 4);
  w.plan.order_e = (int*)take((size_t)nc * 4);
  w.plan.order_i = (int*)take((size_t)nc * 4);
  w.plan.meta = (int*)take(64);
  w.part = (float*)take((size_t)slots * 2 * d.F * d.H * 4);
  w.bytes = o;
  return w;
}

}  // namespace

// bf16: the tile maps of the launches on the forward's GEMM kernel (d_a,
// recompute, dx_sorted, expert outputs: one each, as two of them may run at
// once on two streams)
constexpr int kBwdPlainMaps = 4;

size_t gmm_bwd_scratch_bytes(const Dims& d, int64_t max_rows) {
  const size_t el = d.bf16 ? 2 : 4;
  size_t b = 2 * a256((size_t)(d.G_res + 1) * 4) + 3 * a256((size_t)max_rows * d.F * el) +
             a256((size_t)max_rows * d.F * el);
  if (d.bf16)
    b += kBwdPlainMaps * gmm_scratch_bytes(d) + carve_wgrad(d, max_rows, d.G_res, nullptr).bytes;
  return b;
}

size_t wgrad_sets_scratch_bytes(const Dims& d, int sets, int64_t rows_per_set) {
  return carve_wgrad(d, (int64_t)sets * rows_per_set, sets * d.G_res, nullptr).bytes;
}

hipError_t launch_combine_bwd(const Dims& d, const PassArgs& pa, const LayoutSet& ls,
                              const void* dy, const void* out, const int* roa,
                              long long roa_stride, const float* gate, void* d_out,
                              float* d_gate, int64_t max_rows, int what, hipStream_t s,
                              float* row_gate, const float* dg_part) {
  // a pass of a layer call covers at most its window; the single pass L
  const int ntok = (d.T / d.L) * (pa.ovf != nullptr ? d.L : pa.lw);
  const dim3 grid((ntok + 3) / 4);
  if (d.bf16)
    hipLaunchKernelGGL(combine_bwd_kernel<true>, grid, dim3(256), 0, s, d, pa, ls, dy, out, roa,
                       roa_stride, gate, d_out, d_gate, (long long)max_rows, what, row_gate,
                       dg_part);
  else
    hipLaunchKernelGGL(combine_bwd_kernel<false>, grid, dim3(256), 0, s, d, pa, ls, dy, out, roa,
                       roa_stride, gate, d_out, d_gate, (long long)max_rows, what, row_gate,
                       dg_part);
  return hipGetLastError();
}

hipError_t launch_permute_bwd(const Dims& d, const PassArgs& pa, const LayoutSet& ls,
                              const void* dxs, const int* roa, long long roa_stride, void* dx,
                              int64_t max_rows, hipStream_t s) {
  const int ntok = (d.T / d.L) * (pa.ovf != nullptr ? d.L : pa.lw);
  const dim3 grid((ntok + 3) / 4);
  if (d.bf16)
    hipLaunchKernelGGL(permute_bwd_kernel<true>, grid, dim3(256), 0, s, d, pa, ls, dxs, roa,
                       roa_stride, dx, (long long)max_rows);
  else
    hipLaunchKernelGGL(permute_bwd_kernel<false>, grid, dim3(256), 0, s, d, pa, ls, dxs, roa,
                       roa_stride, dx, (long long)max_rows);
  return hipGetLastError();
}

hipError_t launch_route_bwd(const Dims& d, const int* idx, const float* gate,
                            const float* d_gate, float* d_logits, hipStream_t s) {
  hipLaunchKernelGGL(route_bwd_kernel, dim3((d.T + 3) / 4), dim3(256), 0, s, d, idx, gate, d_gate,
                     d_logits);
  return hipGetLastError();
}

hipError_t launch_wgrad(const Dims& d, int sets, const int* group_offsets, int64_t rows,
                        const int* slot_expert, const void* d_h, const void* x_sorted,
                        const void* d_out, const void* act, float* dwg, float* dwu, float* dwd,
                        int accumulate, void* scratch, hipStream_t s) {
  // plan (rows and chunks per expert over every set's groups), then
  // [dWg ; dWu] = [d_hg | d_hu]^T x_sorted and dWd = d_out^T act, each with
  // the fixed-order sum of split experts' partials
  const int e_res = d.S_res * d.El;
  const int64_t total = (int64_t)sets * rows;
  const WgradScratch wsc = carve_wgrad(d, total, sets * d.G_res, (char*)scratch);
  const int kc = wgrad_kc(d, total);
  const long long nc = wgrad_nc_ub(d, total, kc);
  hipLaunchKernelGGL(wgrad_plan_kernel, dim3(1), dim3(1024), 0, s, wsc.plan, group_offsets,
                     slot_expert, d.G_res, sets, (long long)rows, d.lo_slot, d.e_base, e_res,
                     (long long)rows, kc, (int)nc);
  WgradParams W;
  W.Pm = (const uint16_t*)d_h;
  W.Qm = (const uint16_t*)x_sorted;
  W.C0 = dwg;
  W.C1 = dwu;
  W.part = wsc.part;
  W.c_stride = (size_t)d.F * d.H;
  W.I = 2 * d.F;
  W.J = d.H;
  W.i_split = d.F;
  W.a_rows = (int)total;
  W.plan = wsc.plan;
  W.kc = kc;
  W.slots = wgrad_slots(total, kc);
  W.accumulate = accumulate;
  W.round_blocks = 0;
  W.ni_tiles = W.I / 128;
  W.nj_tiles = W.J / 128;
  WgradParams V = W;
  V.Pm = (const uint16_t*)d_out;
  V.Qm = (const uint16_t*)act;
  V.C0 = V.C1 = dwd;
  V.I = d.H;
  V.J = d.F;
  V.i_split = d.H;
  V.ni_tiles = V.I / 128;
  V.nj_tiles = V.J / 128;
  // long reductions (H >= 2048, both dimensions whole 256-column tiles): the
  // two-group loop on 256 x 256 tiles
  const bool pp = MOE_WGRAD_PP && d.bf16 && d.H >= 2048 && d.H % 256 == 0 && d.F % 256 == 0;
  if (pp) {
    const int nb = bwd_round_blocks(reinterpret_cast<const void*>(wgrad_pp_kernel), 512, 4);
    for (WgradParams* q : {&W, &V}) {
      q->ni_tiles = q->I / 256;
      q->nj_tiles = q->J / 256;
      q->round_blocks = nb;
    }
  }
  for (const WgradParams* q : {&W, &V}) {
    if (pp)
      hipLaunchKernelGGL(wgrad_pp_kernel,
                         dim3(whole_rounds(nc * q->ni_tiles * q->nj_tiles, q->round_blocks)),
                         dim3(512), 0, s, *q);
    else
      hipLaunchKernelGGL(wgrad_kernel, dim3((unsigned)(nc * q->ni_tiles * q->nj_tiles)),
                         dim3(256), 0, s, *q);
    // an expert is split only when it has more than kc rows
    if (kc >= total) continue;
    const long long ij4 = ((long long)q->I * q->J / 4 + 255) / 256;
    hipLaunchKernelGGL(wgrad_reduce_kernel, dim3((unsigned)ij4, (unsigned)e_res), dim3(256), 0, s,
                       *q);
  }
  return hipGetLastError();
}

hipError_t launch_gmm_bwd(const Dims& d, const GemmBwdArgs& a, hipStream_t s) {
  const int e_res = d.S_res * d.El;
  const long long rows = a.max_rows;
  char* ws = (char*)a.scratch;
  const size_t el = d.bf16 ? 2 : 4;
  int* tile_off = (int*)ws;
  ws += a256((size_t)(d.G_res + 1) * 4);
  int* go = (int*)ws;  // the pass's group offsets (bwd_tiles_kernel)
  ws += a256((size_t)(d.G_res + 1) * 4);
  void* d_h = ws;
  ws += 2 * a256((size_t)rows * d.F * el);
  void* act = ws;
  ws += a256((size_t)rows * d.F * el);
  void* d_a = ws;
  ws += a256((size_t)rows * d.F * el);
  char* plain_ws = nullptr;
  const size_t plain_step = d.bf16 ? gmm_scratch_bytes(d) : 0;
  if (d.bf16) {
    plain_ws = ws;
    ws += kBwdPlainMaps * plain_step;
  }
  // a layer call that takes the weight gradients of all its passes at the
  // end keeps each pass's group offsets, d_h and act rows in its own buffers
  if (a.go_out != nullptr) go = a.go_out;
  if (a.d_h_ext != nullptr) d_h = a.d_h_ext;
  if (a.act_ext != nullptr) act = a.act_ext;
  long long lim = (long long)d.T * d.k;
  if (rows < lim) lim = rows;
  hipLaunchKernelGGL(bwd_tiles_kernel, dim3(1), dim3(1024), 0, s, d.G_res, (int)lim, a.pa,
                     a.group_offsets, a.go_stride, go, tile_off);
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
    P.group_offsets = go;
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
  const long long mt_ub = (rows + kBM - 1) / kBM + d.G_res;
  DgradParams P;
  P.group_offsets = go;
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
  // d_a = d_out Wd  (K = H; Wd [H, F] read reduction-major)
  const int nb_km = bwd_round_blocks(reinterpret_cast<const void*>(dgrad_kmajor_kernel), 256, 0);
  const int nb_sw = bwd_round_blocks(reinterpret_cast<const void*>(dgrad_kernel<true>), 256, 1);
  P.A = (const uint16_t*)a.d_out;
  P.B0 = P.B1 = (const uint16_t*)a.wd;
  P.b_stride = (size_t)d.H * d.F;
  P.C = (uint16_t*)d_a;
  P.K = d.H;
  P.k_split = d.H;
  P.Nout = d.F;
  P.n_ntiles = d.F / kBN;
  P.round_blocks = nb_km;
  // with 256-row tiles the data-gradient products run on the forward's
  // kernel reading the weights as stored, reduction-major (each launch with
  // its own tile map); d_a = d_out Wd
  hipError_t pe = launch_gmm_plain_kmajor(d, go, a.slot_expert, a.d_out, rows, a.wd, a.wd, d.H,
                                          (size_t)d.H * d.F, d.H, d.F, d_a, rows, plain_ws, s);
  if (pe == hipErrorNotSupported)
    hipLaunchKernelGGL(dgrad_kmajor_kernel, dim3(whole_rounds(mt_ub * P.n_ntiles, nb_km)),
                       dim3(256), 0, s, P);
  else if (pe != hipSuccess)
    return pe;
  // gate and up products recomputed; SwiGLU backward and the activation
  DgradParams Q = P;
  Q.A = (const uint16_t*)a.x_sorted;
  Q.B0 = (const uint16_t*)a.wg;
  Q.B1 = (const uint16_t*)a.wu;
  Q.b_stride = (size_t)d.F * d.H;
  Q.K = d.H;
  Q.Nout = d.F;
  Q.n_ntiles = d.F / kBN;
  Q.C = nullptr;
  Q.d_a = (const uint16_t*)d_a;
  Q.d_h = (uint16_t*)d_h;
  Q.act = (uint16_t*)act;
  Q.round_blocks = nb_sw;
  pe = launch_gmm_swiglu_recompute(d, go, a.slot_expert, a.x_sorted, rows, a.wg, a.wu, d_a, d_h,
                                   act, rows, plain_ws + 3 * plain_step, s, a.row_gate,
                                   a.dg_part);
  if (pe == hipErrorNotSupported && a.row_gate == nullptr)
    hipLaunchKernelGGL(dgrad_kernel<true>, dim3(whole_rounds(mt_ub * Q.n_ntiles, nb_sw)),
                       dim3(256), 0, s, Q);
  else if (pe != hipSuccess)
    return pe;  // (the gated mode runs on the forward's kernel only)
  // dx_sorted = [d_hg | d_hu] [Wg ; Wu]  (K = 2F; Wg and Wu [F, H] stacked
  // along the reduction and read reduction-major)
  DgradParams X = P;
  X.A = (const uint16_t*)d_h;
  X.B0 = (const uint16_t*)a.wg;
  X.B1 = (const uint16_t*)a.wu;
  X.b_stride = (size_t)d.F * d.H;
  X.C = (uint16_t*)a.dx_sorted;
  X.K = 2 * d.F;
  X.k_split = d.F;
  X.Nout = d.H;
  X.n_ntiles = d.H / kBN;
  // dx_sorted (and the expert outputs) on the side stream, the weight
  // gradients on the caller's: both only read what the launches above wrote,
  // so the data-gradient GEMM fills the weight gradients' uneven last rounds
  SideStream* ss = side_stream();
  std::unique_lock<std::mutex> lock(side_mutex(), std::defer_lock);
  hipStream_t sx = s;
  if (ss != nullptr) {
    lock.lock();
    hipError_t e = hipEventRecord(ss->fork, s);
    if (e == hipSuccess) e = hipStreamWaitEvent(ss->s, ss->fork, 0);
    if (e != hipSuccess) return e;
    sx = ss->s;
  }
  // (a failed launch from here on is reported after the join)
  hipError_t side_err = hipSuccess;
  // dx_sorted = d_hg Wg + d_hu Wu: Wg then Wu [F, H] as stored are the
  // reduction's first and second F rows
  pe = launch_gmm_plain_kmajor(d, go, a.slot_expert, d_h, rows, a.wg, a.wu, d.F,
                               (size_t)d.F * d.H, 2 * d.F, d.H, a.dx_sorted, rows,
                               plain_ws + plain_step, sx);
  if (pe == hipErrorNotSupported)
    hipLaunchKernelGGL(dgrad_kmajor_kernel, dim3(whole_rounds(mt_ub * X.n_ntiles, nb_km)),
                       dim3(256), 0, sx, X);
  else if (pe != hipSuccess)
    side_err = pe;
  pe = hipErrorNotSupported;
  if (a.out_recompute != nullptr)
    pe = launch_gmm_plain(d, go, a.slot_expert, act, rows, a.wd, (size_t)d.H * d.F, d.F, d.H,
                          a.out_recompute, rows, plain_ws + 2 * plain_step, sx);
  if (pe != hipSuccess && pe != hipErrorNotSupported) side_err = pe;
  if (a.out_recompute != nullptr && pe == hipErrorNotSupported) {
    // the expert outputs from the recomputed activation: act Wd^T (K = F,
    // Wd [H, F] K-contiguous)
    DgradParams O = P;
    O.A = (const uint16_t*)act;
    O.B0 = O.B1 = (const uint16_t*)a.wd;
    O.b_stride = (size_t)d.H * d.F;
    O.C = (uint16_t*)a.out_recompute;
    O.K = d.F;
    O.Nout = d.H;
    O.n_ntiles = d.H / kBN;
    const int nb_o = bwd_round_blocks(reinterpret_cast<const void*>(dgrad_kernel<false>), 256, 3);
    O.round_blocks = nb_o;
    hipLaunchKernelGGL(dgrad_kernel<false>, dim3(whole_rounds(mt_ub * O.n_ntiles, nb_o)),
                       dim3(256), 0, sx, O);
  }
  if (a.wgrad && side_err == hipSuccess)
    side_err = launch_wgrad(d, 1, go, rows, a.slot_expert, d_h, a.x_sorted, a.d_out, act, a.dwg,
                            a.dwu, a.dwd, a.accumulate, ws, s);
  if (ss != nullptr) {
    // join even after a failed launch: the caller's stream must not run
    // ahead of the side stream's work
    hipError_t e = hipEventRecord(ss->join, ss->s);
    if (e == hipSuccess) e = hipStreamWaitEvent(s, ss->join, 0);
    if (e != hipSuccess) return e;
  }
  if (side_err != hipSuccess) return side_err;
  return hipGetLastError();
}

}  // namespace moe
