// bf16_fwd.hip -- conventional BF16 attention forward (the baseline).
//
// The pages compare the quantized kernels against BF16 attention ("Fused-
// Softmax shifts an AI attention bottleneck onto faster GPU hardware",
// paragraph 8) and describe the conventional scheme as repeatedly updating a
// reference maximum and rescaling the accumulated results when it grows
// (paragraph 5).  This kernel is that scheme, FlashAttention style:
//   per 64-key step: s = q.k (BF16 MFMA, fp32 accumulate), running max m of
//   s*sigma*log2e, p = exp2(s*sigma*log2e - m), O and l rescaled by
//   exp2(m_old - m_new) when the max grows (by more than 8, so p <= 2^8),
//   O += bf16(p) V (BF16 MFMA), l += sum p; finally O / l.
//
// Mapping to CDNA4 (v_mfma_f32_32x32x16_bf16: lane (r = l%32, h = l/32) holds
// row r, K elements [8h, 8h+8); accumulator lane (c, h) register 4i+j holds
// row 8i+4h+j of column c):
//   * 8 waves per workgroup, 32 queries per wave.  S^T = K Q^T is computed
//     with the K rows of each product permuted so that lane (q, h) receives
//     keys 16t + 8h .. 16t + 8h + 7 of every 16-key chunk t: exactly its A
//     operand of the PV product (no shuffles).
//   * K is streamed by LDS DMA into a 4-slot ring in operand order (one
//     lane-contiguous ds_read_b128 per operand).  V is streamed row-major
//     into a 4-slot ring and read as the PV product's B operand with the
//     transposing LDS read ds_read_b64_tr_b16: within each group of 16 lanes,
//     lane i receives element i % 4 of the 8-byte pieces addressed by lanes
//     4e + i / 4 (e = 0..3), so 16 lanes addressing a 4-key x 16-feature
//     block each receive the 4 keys of one feature (layout measured on
//     gfx950).  The DMA places each row's 16-byte chunks XOR-swizzled by the
//     row index, so that the 4 rows such a group reads fall in distinct
//     quarters of the LDS banks.  Loads run three steps ahead.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"
#include "lds_dma.h"

namespace fsattn {
namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf_b __attribute__((ext_vector_type(2)));
typedef short v4s16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s16 lds_v4s16;

constexpr int BW = 8;         // waves per workgroup
constexpr int BQ = 32;        // queries per wave
constexpr int BQG = BW * BQ;  // queries per workgroup
constexpr int BK = 64;        // keys per step
constexpr int RS = 4;         // K and V ring slots

template <int D> struct BGeo {
  static constexpr int NC = D / 16;          // 16-feature chunks of a score product
  static constexpr int NO = D / 32;          // 32-feature blocks of the PV product
  static constexpr int ROW = 2 * D;          // bytes of a K or V row
  static constexpr int KSLOT = 2 * NC * 1024;  // K operands of a step: 2 key groups x NC chunks
  static constexpr int VSLOT = BK * ROW;       // V rows of a step, row-major, chunks swizzled
  static constexpr int K_OFF = 0;
  static constexpr int V_OFF = K_OFF + RS * KSLOT;
  static constexpr int LDS = V_OFF + RS * VSLOT;
  // DMA per step: one 16-byte load per K operand region (2 NC), VSLOT/1024
  // loads of V rows; waves 0-3 load K, waves 4-7 V, the same count each
  static constexpr int NLOAD = 2 * NC;
  static constexpr int PER_WAVE = NLOAD / 4;
  static_assert(VSLOT / 1024 == NLOAD, "K and V sides issue the same number of loads");
};

// 16-byte chunk c of V row r sits at chunk c ^ vswz(r) of its LDS row: the
// 4 consecutive rows a transposing read covers then use the four 64-byte
// quarters of the 256-byte bank cycle (row r's quarter is (c / 4) ^ (r % 4)
// for D = 128, 2 (r % 2) + ((c / 4) ^ ((r / 2) % 2)) for D = 64)
template <int D> __device__ __forceinline__ constexpr int vswz(int r) {
  return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1);
}

// key (0..31 of a key group) fed to row r of the K operand: accumulator row
// 8i + 4h + j then holds key 16(i/2) + 8h + 4(i%2) + j
__device__ __forceinline__ constexpr int brow_key(int r) {
  return 16 * ((r >> 3) >> 1) + 8 * ((r >> 2) & 1) + 4 * ((r >> 3) & 1) + (r & 3);
}

// two floats -> packed bf16 (RNE)
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  const v2bf_b r = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, r);
}

template <int D>
__global__ void __launch_bounds__(BW * 64, 1) bf16_fwd_kernel(const uint16_t* __restrict__ q,
                                                               const uint16_t* __restrict__ k,
                                                               const uint16_t* __restrict__ v,
                                                               uint16_t* __restrict__ out, int H, int Sq, int Skv,
                                                               float c_log2, int causal,
                                                               const int32_t* __restrict__ q_lens,
                                                               const int32_t* __restrict__ kv_lens) {
  using G = BGeo<D>;
  constexpr int NO = G::NO, NC = G::NC;
  __shared__ __attribute__((aligned(16))) uint8_t smem[G::LDS];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, hh = lane >> 5;
  const int bh = blockIdx.y + blockIdx.z * H;
  // masks as for the fused forward: valid queries / keys of the batch, and the
  // causal limit k <= i + kv_len - q_len; causal workgroups longest first
  const int q_len = q_lens ? min(max(q_lens[blockIdx.z], 0), Sq) : Sq;
  const int kv_len = kv_lens ? min(max(kv_lens[blockIdx.z], 0), Skv) : Skv;
  const int coff = kv_len - q_len;
  const int q0 = (causal ? (int)(gridDim.x - 1 - blockIdx.x) : (int)blockIdx.x) * BQG;
  const int qw0 = q0 + w * BQ;
  int kend = q0 < q_len ? kv_len : 0;  // keys [0, kend) are read
  if (causal) kend = max(min(kend, min(q0 + BQG, q_len) + coff), 0);
  const int ns = (kend + BK - 1) / BK;
  // keys [0, lim) visible to this lane's query; steps from ums on hold a
  // masked key for some row of the wave
  const int lim = (causal && qw0 + n < q_len) ? min(kend, qw0 + n + coff + 1) : kend;
  const int lim_w = (causal && qw0 < q_len) ? min(kend, qw0 + coff + 1) : kend;
  const int ums = max(lim_w, 0) / BK;
  if (ns == 0) {
    // no visible key in the workgroup (uniform): zero rows
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int qq = qw0 + 8 * i + 4 * hh + j;
        if (qq < Sq) {
#pragma unroll
          for (int o = 0; o < NO; ++o) out[((size_t)bh * Sq + qq) * D + 32 * o + n] = 0;
        }
      }
    return;
  }

  // ---- DMA plan: wave w issues loads 4 (w & 3) .. 4 (w & 3) + PER_WAVE - 1 of
  // its side every step, at constant per-lane offsets
  const bool kside = w < 4;
  int lofs[G::PER_WAVE], vofs[G::PER_WAVE];
#pragma unroll
  for (int j = 0; j < G::PER_WAVE; ++j) {
    const int L = G::PER_WAVE * (w & 3) + j;
    if (kside) {
      // K operand region L: key group L / NC, feature chunk L % NC
      const int kg = L / NC, c = L % NC;
      lofs[j] = __builtin_amdgcn_readfirstlane(G::K_OFF + L * 1024);
      vofs[j] = (32 * kg + brow_key(n)) * G::ROW + 32 * c + 16 * hh;
    } else {
      // V rows: load L fills 1024 bytes of the row-major step; LDS chunk c of
      // row r receives global chunk c ^ vswz(r)
      constexpr int CPR = G::ROW / 16;  // chunks per row
      const int r = (L * 1024 + 16 * lane) / G::ROW, c = lane % CPR;
      lofs[j] = __builtin_amdgcn_readfirstlane(G::V_OFF + L * 1024);
      vofs[j] = r * G::ROW + 16 * (c ^ vswz<D>(r));
    }
  }
  const uint64_t base = (uint64_t)(uintptr_t)((kside ? k : v) + (size_t)bh * Skv * D);
  int rem = kend * G::ROW;
  const int stride = BK * G::ROW;
  v4i rc = rsrc(base, rem);
  auto advance = [&]() {
    uint64_t b = ((uint64_t)(uint32_t)rc[1] << 32) | (uint32_t)rc[0];
    b += (uint64_t)stride;
    rc[0] = (int)(uint32_t)b;
    rc[1] = (int)(uint32_t)(b >> 32);
    rem -= stride;
    rc[2] = rem > 0 ? rem : 0;
  };
  const uint32_t lds0 = lds_addr(smem);
  int snext = 0;  // next step to fetch
  auto issue = [&]() {
    const int fill = snext & (RS - 1);
    const uint32_t slot = lds0 + (uint32_t)(kside ? fill * G::KSLOT : fill * G::VSLOT);
    const uint32_t keep = m0_save();
#pragma unroll
    for (int j = 0; j < G::PER_WAVE; ++j) dma_x4(rc, slot, (uint32_t)lofs[j], vofs[j]);
    m0_restore(keep);
    advance();
    ++snext;
  };

  // ---- PV B operand (V, 8 keys of 16-key chunk t for feature 32 o + n, n =
  // lane % 32, keys 8h .. 8h + 7): two transposing reads of 4 keys each.
  // Supplying lane j of a 16-lane group addresses row (key) kq + j / 4,
  // features 16 (group % 2) + 4 (j % 4) .. + 3 of block o.
  const int grp = lane >> 4, jl = lane & 15;
  const int vrow0 = 8 * (grp >> 1) + (jl >> 2);                    // + 16 t + 4 half
  const int vcol = 2 * (16 * (grp & 1) + 4 * (jl & 3));             // bytes within the block's 64
  // the lane's byte offset of block o in a slot (rows 16 t + 4 half + vrow0
  // share vrow0's swizzle), so that each read adds only a constant
  uint32_t voff[NO];
#pragma unroll
  for (int o = 0; o < NO; ++o) {
    const int byte = 64 * o + vcol;  // chunk byte / 16, 8-byte half (byte / 8) % 2
    voff[o] = (uint32_t)(vrow0 * G::ROW + 16 * ((byte >> 4) ^ vswz<D>(vrow0)) + (byte & 15));
  }
  auto v_op = [&](const uint32_t (&vb)[NO], int t, int o) -> v8bf {
    typedef __attribute__((address_space(3))) uint8_t lds_u8;
    const lds_u8* base = (const lds_u8*)(size_t)vb[o];
    const v4s16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s16*)(base + 16 * t * G::ROW));
    const v4s16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s16*)(base + (16 * t + 4) * G::ROW));
    return __builtin_bit_cast(v8bf, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  // ---- Q^T operands (B of S^T): lane (q, h), chunk c: Q[q][16c + 8h .. +8]
  v8bf qB[NC];
  {
    const int qrow = min(qw0 + n, Sq - 1);
    const uint16_t* qp = q + ((size_t)bh * Sq + qrow) * D;
#pragma unroll
    for (int c = 0; c < NC; ++c) qB[c] = __builtin_bit_cast(v8bf, *reinterpret_cast<const uint4*>(qp + 16 * c + 8 * hh));
  }
  // the Q loads land before any DMA is issued: their first use is inside the
  // step loop, and the waits the compiler places before a first use would
  // otherwise sit in the loop body, where they count the step's own DMA
  // loads as well (down to vmcnt 0: every step waited for the loads it had
  // just issued).  The empty statements use the registers, so the compiler
  // waits for the loads here, ahead of the DMA statements.
#pragma unroll
  for (int c = 0; c < NC; ++c) asm volatile("" ::"v"(qB[c]));

  v16f O[NO];
#pragma unroll
  for (int o = 0; o < NO; ++o)
#pragma unroll
    for (int e = 0; e < 16; ++e) O[o][e] = 0.0f;
  // byte address of lane ^ 32 (the other half of the query's keys), for ds_bpermute
  const int xhalf = (lane ^ 32) << 2;
  float m = -INFINITY;  // running max of query n (scaled, log2 units), lanes n and n + 32 agree
  float lsum = 0.0f;    // this lane's share of the row sum

  // prologue: steps 0..2 in flight
  for (int s = 0; s < 3; ++s) issue();

  for (int u = 0; u < ns; ++u) {
    // steps <= u landed (u + 1 and u + 2 may be in flight); after the barrier
    // the loads of step u + 3 reuse the slots of step u - 1, which every wave
    // finished reading before it
    wait_vm<2 * G::PER_WAVE>();
    barrier();
    issue();
    const int slot = u & (RS - 1);

    // ---- S^T = K Q^T for the step's two key groups
    const uint8_t* ks = smem + G::K_OFF + slot * G::KSLOT;
    v16f S[2];
#pragma unroll
    for (int kg = 0; kg < 2; ++kg) {
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const v8bf a = __builtin_bit_cast(v8bf, *reinterpret_cast<const uint4*>(ks + (kg * NC + c) * 1024 + 16 * lane));
        if (c == 0) {
          v16f z;
#pragma unroll
          for (int e = 0; e < 16; ++e) z[e] = 0.0f;
          S[kg] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qB[0], z, 0, 0, 0);
        } else {
          S[kg] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qB[c], S[kg], 0, 0, 0);
        }
      }
    }
    // lane (q, h), register 4i + j of key group kg holds key 32 kg + 16(i/2) + 8h + 4(i%2) + j
    if (u >= ums) {
      const int nk = lim - u * BK;  // this lane's visible keys of the step
#pragma unroll
      for (int kg = 0; kg < 2; ++kg)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int i = e >> 2, j = e & 3;
          const int key = 32 * kg + 16 * (i >> 1) + 8 * hh + 4 * (i & 1) + j;
          if (key >= nk) S[kg][e] = -INFINITY;
        }
    }
    // row maximum with IEEE 754-2019 maximum (v_maximum3_f32): unlike fmaxf
    // it needs no quieting of its inputs, and scores are finite or -inf
    float mx = __builtin_elementwise_maximum(S[0][0], S[0][1]);
#pragma unroll
    for (int i = 2; i < 32; i += 2)
      mx = __builtin_elementwise_maximum(__builtin_elementwise_maximum(mx, S[i >> 4][i & 15]), S[i >> 4][(i + 1) & 15]);
    mx *= c_log2;
    mx = __builtin_fmaxf(mx, __int_as_float(__builtin_amdgcn_ds_bpermute(xhalf, __float_as_int(mx))));
    const float mnew = __builtin_fmaxf(m, mx);
    // the reference moves only when some row's maximum grows by more than 8
    // (a factor of 256; FlashAttention-4's conditional rescale): below that
    // p stays at most 2^8, which bf16 and the fp32 sums carry exactly as
    // well, and most steps skip the rescale (4-5 % of the kernel's time)
    if (__ballot(mnew > m + 8.0f) != 0) {
      // rescale O and l by exp2(m_old - m_new)
      const float alpha = __builtin_amdgcn_exp2f(m - mnew);
      lsum *= alpha;
      int base4 = hh << 4;  // byte address of lane 4h
      asm volatile("" : "+v"(base4));
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float r = __int_as_float(__builtin_amdgcn_ds_bpermute(base4 + 4 * (8 * i + j), __float_as_int(alpha)));
#pragma unroll
          for (int o = 0; o < NO; ++o) O[o][4 * i + j] *= r;
        }
      m = mnew;
    }
    // p = exp2(s c - m), l += p, P operands of the four 16-key chunks (a row
    // that has seen no key yet keeps m = -inf: its masked scores give p = 0)
    const float mref = m > -INFINITY ? m : 0.0f;
    // l sums the bf16 p that the PV product uses, two at a time (v_dot2 with
    // ones), in four independent chains
    uint32_t pw[16];
    float lp[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kg = 0; kg < 2; ++kg)
#pragma unroll
      for (int e = 0; e < 16; e += 2) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(S[kg][e], c_log2, -mref));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(S[kg][e + 1], c_log2, -mref));
        const int i = 8 * kg + e / 2;
        pw[i] = pk_bf16(p0, p1);
        lp[i & 3] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2bf_b, pw[i]),
                                                    __builtin_bit_cast(v2bf_b, 0x3F803F80u), lp[i & 3], false);
      }
    lsum += (lp[0] + lp[1]) + (lp[2] + lp[3]);
    // ---- O += P V: chunk t = 2 kg + (i / 2) holds registers 8t .. 8t + 7
    const uint32_t vslot = lds0 + (uint32_t)(G::V_OFF + slot * G::VSLOT);
    uint32_t vb[NO];
#pragma unroll
    for (int o = 0; o < NO; ++o) vb[o] = vslot + voff[o];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const v8bf pa = __builtin_bit_cast(v8bf, uint4{pw[4 * t], pw[4 * t + 1], pw[4 * t + 2], pw[4 * t + 3]});
#pragma unroll
      for (int o = 0; o < NO; ++o) O[o] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa, v_op(vb, t, o), O[o], 0, 0, 0);
    }
  }
  wait_vm<0>();  // loads past the end are still in flight

  // ---- O / l -> bf16: lane (d % 32, h) register 4i + j holds query 8i + 4h + j
  const float ltot = lsum + __shfl_xor(lsum, 32, 64);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int qi = 8 * i + 4 * hh + j;
      const float lq = __shfl(ltot, qi, 64);
      const int qq = qw0 + qi;
      if (qq < Sq) {
        // rows past q_len and rows that saw no key are stored as 0
        const bool live = qq < q_len && lq > 0.0f;
        const float inv = live ? 1.0f / lq : 0.0f;
        uint16_t* orow = out + ((size_t)bh * Sq + qq) * D;
#pragma unroll
        for (int o = 0; o < NO; ++o) {
          uint32_t uo = live ? __float_as_uint(O[o][4 * i + j] * inv) : 0u;
          uo = (uo + 0x7FFFu + ((uo >> 16) & 1u)) >> 16;  // RNE to bf16 (finite values)
          orow[32 * o + n] = (uint16_t)uo;
        }
      }
    }
}

}  // namespace

hipError_t launch_bf16_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* out, int B, int H,
                           int Sq, int Skv, int D, float softmax_scale, int causal, const int32_t* q_lens,
                           const int32_t* kv_lens, hipStream_t stream) {
  const float c_log2 = softmax_scale * 1.4426950408889634f;
  dim3 grid((unsigned)((Sq + BQG - 1) / BQG), (unsigned)H, (unsigned)B);
  if (D == 128)
    hipLaunchKernelGGL(bf16_fwd_kernel<128>, grid, dim3(BW * 64), 0, stream, q, k, v, out, H, Sq, Skv, c_log2,
                       causal, q_lens, kv_lens);
  else
    hipLaunchKernelGGL(bf16_fwd_kernel<64>, grid, dim3(BW * 64), 0, stream, q, k, v, out, H, Sq, Skv, c_log2,
                       causal, q_lens, kv_lens);
  return hipGetLastError();
}

}  // namespace fsattn
