// Prefill expert FFN: grouped GEMMs on the bf16 matrix cores.
//
// Prefill batches are large enough that each expert's pairs form a real
// matrix (a few hundred rows per expert), so the FFN is a grouped GEMM
// rather than matrix-vector work (the fork README, "Quant types", pairs
// matrix-matrix kernels with prefill).  Per expert: h = silu(X Wg^T) *
// (X Wu^T) with X the expert's gathered token rows, then y = h Wd^T.
//
// Tiles.  A workgroup (4 wavefronts, 2 x 2) computes a 128 x 128 output
// tile of one expert with v_mfma_f32_32x32x16_bf16; each wavefront owns
// 64 x 64 (2 x 2 MFMA tiles).  Per K step of 64: the A tile (gathered
// activation rows, bf16) and the B tile (weight rows, Q4_0/Q8_0 blocks
// dequantised to bf16 = round-to-nearest-even of d * q) are written to LDS
// (rows padded by 16 B so the 16-byte fragment reads do not collide in the
// banks), while the next step's global loads are already in flight.
//
// Gate/up tiles hold 64 gate rows and the 64 up rows of the same
// intermediate indices, so SwiGLU is applied in the accumulator registers.
#include "device_common.h"
#include "ffn.h"
#include "route_common.h"

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kPBM = 128, kPBN = 128, kPBK = 64;
constexpr int kPLD = kPBK + 8;  // LDS row stride in bf16 elements

// ------------------------------------------------------------ tile list
// One workgroup: for every expert with pairs, the 128-row tiles
// (expert, first row) in expert order; tiles[n] for n >= count is unused.
__global__ __launch_bounds__(256) void prefill_tiles_kernel(const int32_t* __restrict__ offsets, int E,
                                                            int2* __restrict__ tiles, int* __restrict__ count) {
  __shared__ int s_n[kMaxE];
  __shared__ int s_base[kMaxE];
  __shared__ int s_wave[4];
  for (int e = threadIdx.x; e < E; e += 256) {
    const int m = offsets[e + 1] - offsets[e];
    s_n[e] = (m + kPBM - 1) / kPBM;
  }
  __syncthreads();
  const int total = block_exclusive_scan<256>(s_n, s_base, E, s_wave);
  for (int e = threadIdx.x; e < E; e += 256)
    for (int j = 0; j < s_n[e]; ++j) tiles[s_base[e] + j] = make_int2(e, j * kPBM);
  if (threadIdx.x == 0) *count = total;
}

// --------------------------------------------------------- B tile staging
// Thread t stages half a K step (one 32-weight block) of weight row t / 2.
template <int QT>
struct BStage {
  uint32_t w[QT == MOE_QTYPE_Q8_0 ? 8 : 4];
  float d;
  __device__ __forceinline__ void load(const uint8_t* row, int b) {
    const uint8_t* q = block_quants<QT>(row, b);
    const uint4 v0 = *reinterpret_cast<const uint4*>(q);
    w[0] = v0.x; w[1] = v0.y; w[2] = v0.z; w[3] = v0.w;
    if constexpr (QT == MOE_QTYPE_Q8_0) {
      const uint4 v1 = *reinterpret_cast<const uint4*>(q + 16);
      w[4] = v1.x; w[5] = v1.y; w[6] = v1.z; w[7] = v1.w;
    }
    d = block_scale<QT>(row, b);
  }
  // 32 weights d*q (Q8_0) or d*(q-8) (Q4_0), exact in fp32, rounded to bf16.
  __device__ __forceinline__ void store(__bf16* dst) const {
    bf16x8 o[4];
    if constexpr (QT == MOE_QTYPE_Q8_0) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) o[i / 2][(i & 1) * 4 + j] = (__bf16)(d * (float)(int8_t)(w[i] >> (8 * j)));
    } else {
      const float d8 = -8.0f * d;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int byte = (w[i] >> (8 * j)) & 0xFF;
          o[i / 2][(i & 1) * 4 + j] = (__bf16)fmaf(d, (float)(byte & 0xF), d8);
          o[2 + i / 2][(i & 1) * 4 + j] = (__bf16)fmaf(d, (float)(byte >> 4), d8);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<bf16x8*>(dst + 8 * i) = o[i];
  }
};

// One wavefront's 64 x 64 of the 128 x 128 tile: acc[mt][nt] for the 32 x 32
// MFMA tiles; a_row0 / b_row0 select the wavefront's rows in the LDS tiles.
__device__ __forceinline__ void mma_k64(const __bf16 (*sA)[kPLD], const __bf16 (*sB)[kPLD], int a_row0,
                                        const int (&b_row0)[2], f32x16 (&acc)[2][2]) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int ks = 0; ks < kPBK / 16; ++ks) {
    const int kc = 16 * ks + 8 * (lane >> 5);
    bf16x8 a[2], b[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) a[mt] = *reinterpret_cast<const bf16x8*>(&sA[a_row0 + 32 * mt + (lane & 31)][kc]);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) b[nt] = *reinterpret_cast<const bf16x8*>(&sB[b_row0[nt] + (lane & 31)][kc]);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mt], b[nt], acc[mt][nt], 0, 0, 0);
  }
}

// ------------------------------------------------------ gate/up + SwiGLU
template <int QT>
__global__ __launch_bounds__(256) void prefill_gateup_kernel(FfnParams p, const __bf16* __restrict__ x,
                                                             const int2* __restrict__ tiles,
                                                             const int* __restrict__ n_tiles,
                                                             __bf16* __restrict__ hout) {
  __shared__ __bf16 sA[kPBM][kPLD];
  __shared__ __bf16 sB[kPBN][kPLD];
  const int ntn = p.I / 64;
  const int mt_i = blockIdx.x / ntn, nt_i = blockIdx.x - mt_i * ntn;
  if (mt_i >= *n_tiles) return;
  const int2 tl = tiles[mt_i];
  const int e = tl.x, m0 = tl.y;
  const int slot = p.slot_table[e];
  const int pbeg = p.offsets[e];
  const int rows = min(kPBM, p.offsets[e + 1] - pbeg - m0);
  const int i0 = nt_i * 64;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  if (slot < 0 || slot >= p.n_slots) {
    if (tid == 0) atomicCAS(p.err, 0, e + 1);
    for (int idx = tid; idx < rows * 64; idx += 256)
      hout[(size_t)(pbeg + m0 + idx / 64) * p.I + i0 + idx % 64] = (__bf16)NAN;
    return;
  }
  // A: thread t moves 16-byte chunks c = t + 256 j: row c / 8, chunk c % 8
  const __bf16* asrc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = (tid + 256 * j) >> 3;
    asrc[j] = r < rows ? x + (size_t)(p.sorted_pairs[pbeg + m0 + r] / p.k) * p.H + 8 * (tid & 7) : nullptr;
  }
  // B: thread t stages weight row t / 2 (gate rows 0..63, up rows 64..127), block half t & 1
  const int brow = tid >> 1, bhalf = tid & 1;
  const uint8_t* base = p.pool + (size_t)slot * p.slot_bytes;
  const uint8_t* wrow = base + (brow < 64 ? slot_gate_off(QT, p.H, p.I) : slot_up_off(QT, p.H, p.I)) +
                        (size_t)(i0 + (brow & 63)) * row_bytes(QT, p.H);
  const int wm = wave >> 1, wn = wave & 1;
  const int b_row0[2] = {32 * wn, 64 + 32 * wn};
  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f32x16{};
  uint4 areg[4];
  BStage<QT> breg;
  auto fetch = [&](int kk) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      areg[j] = asrc[j] ? *reinterpret_cast<const uint4*>(asrc[j] + kk * kPBK) : make_uint4(0, 0, 0, 0);
    breg.load(wrow, kk * 2 + bhalf);
  };
  const int nk = p.H / kPBK;
  fetch(0);
  for (int kk = 0; kk < nk; ++kk) {
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = tid + 256 * j;
      *reinterpret_cast<uint4*>(&sA[c >> 3][8 * (c & 7)]) = areg[j];
    }
    breg.store(&sB[brow][32 * bhalf]);
    __syncthreads();
    if (kk + 1 < nk) fetch(kk + 1);
    mma_k64(sA, sB, 64 * wm, b_row0, acc);
  }
  // SwiGLU in registers: acc[mt][0] holds gate, acc[mt][1] up at the same (m, n)
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = 64 * wm + 32 * mt + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      if (m < rows) {
        const float g = acc[mt][0][r], u = acc[mt][1][r];
        hout[(size_t)(pbeg + m0 + m) * p.I + i0 + 32 * wn + (lane & 31)] = (__bf16)(g / (1.0f + expf(-g)) * u);
      }
    }
  }
}

// ------------------------------------------------------------------ down
template <int QT>
__global__ __launch_bounds__(256) void prefill_down_kernel(FfnParams p, const __bf16* __restrict__ hin,
                                                           const int2* __restrict__ tiles,
                                                           const int* __restrict__ n_tiles) {
  __shared__ __bf16 sA[kPBM][kPLD];
  __shared__ __bf16 sB[kPBN][kPLD];
  const int ntn = p.H / kPBN;
  const int mt_i = blockIdx.x / ntn, nt_i = blockIdx.x - mt_i * ntn;
  if (mt_i >= *n_tiles) return;
  const int2 tl = tiles[mt_i];
  const int e = tl.x, m0 = tl.y;
  const int slot = p.slot_table[e];
  const int pbeg = p.offsets[e];
  const int rows = min(kPBM, p.offsets[e + 1] - pbeg - m0);
  const int n0 = nt_i * kPBN;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  if (slot < 0 || slot >= p.n_slots) {
    for (int idx = tid; idx < rows * kPBN; idx += 256)
      p.y[(size_t)p.sorted_pairs[pbeg + m0 + idx / kPBN] * p.H + n0 + idx % kPBN] = NAN;
    return;
  }
  const __bf16* asrc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = (tid + 256 * j) >> 3;
    asrc[j] = r < rows ? hin + (size_t)(pbeg + m0 + r) * p.I + 8 * (tid & 7) : nullptr;
  }
  const int brow = tid >> 1, bhalf = tid & 1;
  const uint8_t* wrow = p.pool + (size_t)slot * p.slot_bytes + slot_down_off(QT, p.H, p.I) +
                        (size_t)(n0 + brow) * row_bytes(QT, p.I);
  const int wm = wave >> 1, wn = wave & 1;
  const int b_row0[2] = {64 * wn, 64 * wn + 32};
  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f32x16{};
  uint4 areg[4];
  BStage<QT> breg;
  auto fetch = [&](int kk) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      areg[j] = asrc[j] ? *reinterpret_cast<const uint4*>(asrc[j] + kk * kPBK) : make_uint4(0, 0, 0, 0);
    breg.load(wrow, kk * 2 + bhalf);
  };
  const int nk = p.I / kPBK;
  fetch(0);
  for (int kk = 0; kk < nk; ++kk) {
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = tid + 256 * j;
      *reinterpret_cast<uint4*>(&sA[c >> 3][8 * (c & 7)]) = areg[j];
    }
    breg.store(&sB[brow][32 * bhalf]);
    __syncthreads();
    if (kk + 1 < nk) fetch(kk + 1);
    mma_k64(sA, sB, 64 * wm, b_row0, acc);
  }
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = 64 * wm + 32 * mt + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      if (m < rows) {
        float* yrow = p.y + (size_t)p.sorted_pairs[pbeg + m0 + m] * p.H + n0 + 64 * wn + (lane & 31);
        yrow[0] = acc[mt][0][r];
        yrow[32] = acc[mt][1][r];
      }
    }
  }
}

bool prefill_mfma_supported(int H, int I) { return H % kPBN == 0 && I % 64 == 0 && H % kPBK == 0; }

size_t prefill_ws_bytes(int T, int k, int I, int E) {
  const size_t P = (size_t)T * k;
  const size_t max_tiles = P / kPBM + (size_t)E + 1;
  return 256 + ((max_tiles * sizeof(int2) + 255) / 256) * 256 + P * I * sizeof(__bf16);
}

int launch_ffn_prefill(moe_ctx* ctx, const FfnParams& p, const void* x, void* ws, hipStream_t s) {
  const size_t P = (size_t)p.T * p.k;
  const int max_tiles = (int)(P / kPBM) + p.E + 1;
  int* count = (int*)ws;
  int2* tiles = (int2*)((char*)ws + 256);
  __bf16* hbuf = (__bf16*)((char*)ws + 256 + ((max_tiles * sizeof(int2) + 255) / 256) * 256);
  {
    KernelTimer timer(ctx, "prefill_tiles", s);
    launch(prefill_tiles_kernel, 1, 256, 0, s, p.offsets, p.E, tiles, count);
  }
  int rc = check_launch("prefill_tiles_kernel");
  if (rc) return rc;
  {
    KernelTimer timer(ctx, "ffn_gateup", s);
    const unsigned grid = (unsigned)max_tiles * (p.I / 64);
    if (p.qtype == MOE_QTYPE_Q4_0)
      launch(prefill_gateup_kernel<MOE_QTYPE_Q4_0>, grid, 256, 0, s, p, (const __bf16*)x, tiles, count, hbuf);
    else
      launch(prefill_gateup_kernel<MOE_QTYPE_Q8_0>, grid, 256, 0, s, p, (const __bf16*)x, tiles, count, hbuf);
  }
  if ((rc = check_launch("prefill_gateup_kernel"))) return rc;
  {
    KernelTimer timer(ctx, "ffn_down", s);
    const unsigned grid = (unsigned)max_tiles * (p.H / kPBN);
    if (p.qtype == MOE_QTYPE_Q4_0)
      launch(prefill_down_kernel<MOE_QTYPE_Q4_0>, grid, 256, 0, s, p, hbuf, tiles, count);
    else
      launch(prefill_down_kernel<MOE_QTYPE_Q8_0>, grid, 256, 0, s, p, hbuf, tiles, count);
  }
  return check_launch("prefill_down_kernel");
}

}  // namespace moe
