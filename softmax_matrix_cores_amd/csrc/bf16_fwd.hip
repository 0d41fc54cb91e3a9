// bf16_fwd.hip -- conventional BF16 attention forward (the baseline).
//
// The pages compare the quantized kernels against BF16 attention ("Fused-
// Softmax shifts an AI attention bottleneck onto faster GPU hardware",
// paragraph 8) and describe the conventional scheme as repeatedly updating a
// reference maximum and rescaling the accumulated results when it grows
// (paragraph 5).  This kernel is that scheme, FlashAttention style:
//   per 64-key step: s = q.k (BF16 MFMA, fp32 accumulate), running max m of
//   s*sigma*log2e, p = exp2(s*sigma*log2e - m), O and l rescaled by
//   exp2(m_old - m_new) when the max grows, O += bf16(p) V (BF16 MFMA),
//   l += sum p; finally O / l.
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
//     into a 3-slot staging ring, and the workgroup transposes each step once
//     (4x4 blocks of 16-bit elements in registers) into V^T operands in
//     operand order, double buffered.  Loads run three steps ahead.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"
#include "lds_dma.h"

namespace fsattn {
namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf_b __attribute__((ext_vector_type(2)));

constexpr int BW = 8;         // waves per workgroup
constexpr int BQ = 32;        // queries per wave
constexpr int BQG = BW * BQ;  // queries per workgroup
constexpr int BK = 64;        // keys per step
constexpr int KR = 4;         // K ring slots
constexpr int VR = 3;         // V staging ring slots

template <int D> struct BGeo {
  static constexpr int NC = D / 16;          // 16-feature chunks of a score product
  static constexpr int NO = D / 32;          // 32-feature blocks of the PV product
  static constexpr int ROW = 2 * D;          // bytes of a K or V row
  static constexpr int KSLOT = 2 * NC * 1024;  // K operands of a step: 2 key groups x NC chunks
  static constexpr int VSLOT = BK * ROW;       // V rows of a step, row-major
  static constexpr int VT = 4 * NO * 1024;     // V^T operands: 4 key chunks x NO blocks
  static constexpr int K_OFF = 0;
  static constexpr int VS_OFF = K_OFF + KR * KSLOT;
  static constexpr int VT_OFF = VS_OFF + VR * VSLOT;
  static constexpr int LDS = VT_OFF + 2 * VT;
  // DMA per step: one 16-byte load per K operand region (2 NC), VSLOT/1024
  // loads of V rows; waves 0-3 load K, waves 4-7 V, the same count each
  static constexpr int NLOAD = 2 * NC;
  static constexpr int PER_WAVE = NLOAD / 4;
  static_assert(VSLOT / 1024 == NLOAD, "K and V sides issue the same number of loads");
};

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
      // V rows: load L covers 1024 bytes of the row-major step
      lofs[j] = __builtin_amdgcn_readfirstlane(G::VS_OFF + L * 1024);
      vofs[j] = L * 1024 + 16 * lane;
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
  int kfill = 0, vfill = 0;  // its K and V ring slots
  auto issue = [&]() {
    const uint32_t slot = lds0 + (uint32_t)(kside ? kfill * G::KSLOT : vfill * G::VSLOT);
    const uint32_t keep = m0_save();
#pragma unroll
    for (int j = 0; j < G::PER_WAVE; ++j) dma_x4(rc, slot, (uint32_t)lofs[j], vofs[j]);
    m0_restore(keep);
    advance();
    ++snext;
    kfill = kfill == KR - 1 ? 0 : kfill + 1;
    vfill = vfill == VR - 1 ? 0 : vfill + 1;
  };

  // ---- transpose of one step's V rows (staging slot vs) into V^T operands
  // (buffer vt): thread item (key quad kq, feature quad dq)
  auto transpose = [&](int vs, int vt) {
    const uint8_t* st = smem + G::VS_OFF + vs * G::VSLOT;
    uint8_t* dst = smem + G::VT_OFF + vt * G::VT;
    constexpr int ITEMS = 16 * (D / 4);
#pragma unroll
    for (int it = tid; it < ITEMS; it += BW * 64) {
      const int kq = it / (D / 4), dq = it % (D / 4);
      uint2 r[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) r[e] = *reinterpret_cast<const uint2*>(st + (4 * kq + e) * G::ROW + 8 * dq);
      // key k = 4 kq + e, feature d = 4 dq + f: chunk t = kq / 4, lane half
      // (kq % 4) / 2, element 4 (kq % 2) + e of lane (h, d % 32)
      const int t = kq >> 2, h2 = (kq >> 1) & 1;
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const int d = 4 * dq + f;
        const uint32_t sel = (f & 1) ? 0x07060302u : 0x05040100u;  // high or low halves of (b, a)
        const uint32_t w0 = (f < 2) ? r[0].x : r[0].y, w1 = (f < 2) ? r[1].x : r[1].y;
        const uint32_t w2 = (f < 2) ? r[2].x : r[2].y, w3 = (f < 2) ? r[3].x : r[3].y;
        const uint2 o2 = make_uint2(__builtin_amdgcn_perm(w1, w0, sel), __builtin_amdgcn_perm(w3, w2, sel));
        const int region = t * NO + (d >> 5);
        *reinterpret_cast<uint2*>(dst + region * 1024 + (32 * h2 + (d & 31)) * 16 + 8 * (kq & 1)) = o2;
      }
    }
  };

  // ---- Q^T operands (B of S^T): lane (q, h), chunk c: Q[q][16c + 8h .. +8]
  v8bf qB[NC];
  {
    const int qrow = min(qw0 + n, Sq - 1);
    const uint16_t* qp = q + ((size_t)bh * Sq + qrow) * D;
#pragma unroll
    for (int c = 0; c < NC; ++c) qB[c] = __builtin_bit_cast(v8bf, *reinterpret_cast<const uint4*>(qp + 16 * c + 8 * hh));
  }

  v16f O[NO];
#pragma unroll
  for (int o = 0; o < NO; ++o)
#pragma unroll
    for (int e = 0; e < 16; ++e) O[o][e] = 0.0f;
  float m = -INFINITY;  // running max of query n (scaled, log2 units), lanes n and n + 32 agree
  float lsum = 0.0f;    // this lane's share of the row sum

  // prologue: steps 0..2 in flight; step 0 transposed before the loop
  for (int s = 0; s < 3; ++s) issue();
  wait_vm<2 * G::PER_WAVE>();
  barrier();
  transpose(0, 0);
  int kread = 0, vstage = 1;  // K ring slot of step u; staging slot of step u + 1

  for (int u = 0; u < ns; ++u) {
    // steps <= u + 1 landed; after the barrier the loads of step u + 3 reuse
    // the K slot of step u - 1 and the staging slot of step u, both consumed
    wait_vm<G::PER_WAVE>();
    wait_lgkm0();  // the previous step's transpose writes (ds_write) are done
    barrier();
    issue();
    transpose(vstage, (u + 1) & 1);

    // ---- S^T = K Q^T for the step's two key groups
    const uint8_t* ks = smem + G::K_OFF + kread * G::KSLOT;
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
    float mx = -INFINITY;
#pragma unroll
    for (int kg = 0; kg < 2; ++kg)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = __builtin_fmaxf(mx, S[kg][e]);
    mx *= c_log2;
    mx = __builtin_fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mnew = __builtin_fmaxf(m, mx);
    if (__ballot(mnew > m) != 0) {
      // the reference grows: rescale O and l by exp2(m_old - m_new)
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
    uint32_t pw[16];
#pragma unroll
    for (int kg = 0; kg < 2; ++kg)
#pragma unroll
      for (int e = 0; e < 16; e += 2) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(S[kg][e], c_log2, -mref));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(S[kg][e + 1], c_log2, -mref));
        lsum += p0 + p1;
        pw[8 * kg + e / 2] = pk_bf16(p0, p1);
      }
    // ---- O += P V: chunk t = 2 kg + (i / 2) holds registers 8t .. 8t + 7
    const uint8_t* vt = smem + G::VT_OFF + (u & 1) * G::VT;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const v8bf pa = __builtin_bit_cast(v8bf, uint4{pw[4 * t], pw[4 * t + 1], pw[4 * t + 2], pw[4 * t + 3]});
#pragma unroll
      for (int o = 0; o < NO; ++o) {
        const v8bf b = __builtin_bit_cast(v8bf, *reinterpret_cast<const uint4*>(vt + (t * NO + o) * 1024 + 16 * lane));
        O[o] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa, b, O[o], 0, 0, 0);
      }
    }
    kread = kread == KR - 1 ? 0 : kread + 1;
    vstage = vstage == VR - 1 ? 0 : vstage + 1;
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
