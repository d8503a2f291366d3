// kvq_extend.hip -- extend (chunked-prefill) attention over the bf16 workspace.
//
// What it computes ("SGLang's 4-bit KV cache: the 56% is exact, the 1.78x is
// untested", Figure 2 caption: the chunked-prefill / extend path dequantizes
// the cached prefix into a reused workspace and attends over prefix plus
// current chunk): the workspace holds bf16 K and V rows for tokens
// [0, prefix_len + chunk_len) -- the prefix from kvq_dequant_prefix, then the
// chunk's own K/V -- and chunk query i (sequence position prefix_len + i)
// attends causally to keys 0 .. prefix_len + i.
//
// Structure: the (chunk token, query head) pairs of one KV head are flattened
// into query rows r = i * G + h; a workgroup takes 16 consecutive rows per
// wavefront (the MFMA's column dimension) -- 12 wavefronts, 192 rows, in the
// paged variant, 8 wavefronts, 128 rows, over the workspace -- and walks the
// keys its rows can see in 32-token steps.  Each step's K rows and V rows are
// staged once in LDS, by the first 8 wavefronts, and read by all.  LDS holds
// four steps (step s in buffer s mod 4): one step is computed while the next
// is staged, its global loads in flight in registers; on the paged variant's
// prefix steps, two steps are computed per barrier while the next two are
// staged, from two sets of loads issued a pair of steps ahead.  At head dim
// 256 the workgroup fills a compute unit (three wavefronts per SIMD in the
// paged variant, two over the workspace; 140 KB of LDS), so every wavefront
// of the unit shares one staging:
//   QK  S^T[token][row] = K[token][ch] Q^T[ch][row] on v_mfma_f32_16x16x32_bf16
//       (bf16 K and q exactly, fp32 accumulation);
//   online softmax in base 2 per row, lazily rescaled as in decode;
//   PV  O^T[ch][row] += V^T[ch][token] P^T[token][row], P split into bf16
//       hi + lo parts (two MFMAs) so the product keeps ~16 bits of each p.
//
// Paged variant (SRC = the cache format): the same kernel reads the prefix
// straight from the 4-bit pages instead of a bf16 workspace -- the fused
// extend that needs no workspace -- and the chunk's own K/V from bf16 rows.
// Prefix codes are expanded to bf16 exactly while staged (NVFP4 e2m1 * e4m3;
// INT4 q) and the remaining factor of each token (NVFP4: the global scale;
// INT4: the token's scale; chunk tokens: 1) is staged per token and applied
// to its score (K) and to its probability in the PV product (V).  The steps
// whose keys all lie in the prefix run in fp16 instead: codes expanded
// exactly to fp16, q scaled per row by a power of two into fp16's range, QK
// and PV on v_mfma_f32_16x16x32_f16 with p in fp16 (one PV MFMA).  NVFP4's
// factors there are the layer's two global scales, applied to the score and,
// once, to the output accumulators; INT4's value scale rides on p, kept in
// fp16's range by a running max that bounds p * scale.
#include <mutex>
#include <type_traits>

#include "kvq_device.h"
#include "kvq_launch.h"

namespace kvq {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

constexpr int kExtStagers = 512;  // threads that stage K/V (wavefronts 0..7)
constexpr int kExtStep = 32;   // key tokens per step
constexpr int kExtBufs = 4;    // staged steps in LDS (step s in buffer s mod 4)
constexpr int kExtFlush = 32;  // steps an MFMA accumulator runs before it is added into the total
static constexpr float kExtLog2e = 1.4426950408889634f;
static constexpr float kExtLn2 = 0.6931471805599453f;
static constexpr float kExtSlack = 8.0f;

// LDS layout, chosen from measured bank-conflict counts of each access
// pattern on gfx950: K and V are both staged by token row, D/2 + 8 dwords
// apart.  With that stride the QK operand reads (16-byte, lane (j, n) reading
// column j of row n) and the PV operand reads -- transposing 8-byte reads
// (ds_read_b64_tr_b16), where the 16 lanes of a group each name 4 channels of
// one token row and every lane receives one channel of 4 tokens -- are
// conflict-free, and the staging writes (16-byte segments, whole rows per
// half-wavefront) run as fast as a linear store.  No transposition in
// registers: V rows are copied like K rows.
template <int D>
struct ExtLds {
  static constexpr int KPD = D / 2 + 8;  // dwords per staged K or V row
  static constexpr int KB = kExtStep * KPD * 4;
  static constexpr int VB = KB;
  static constexpr int BUF = KB + VB + 2 * kExtStep * 4;  // + per-token K and V factors
  static constexpr int TOTAL = kExtBufs * BUF;
};

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t* lds_v4i16_ptr;
// LDS pointers typed in the LDS address space: every offset into the
// staging buffers is 32-bit arithmetic by construction, without relying on
// the compiler to infer the address space of generic pointers
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) float lds_f32;
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4;

constexpr int kExtWorkspace = 0;  // SRC: every key from the bf16 workspace (else the cache format)

// Wavefronts per workgroup, 16 query rows each.  The paged variant runs 12,
// three per SIMD: the first 8 stage and compute, the other 4 compute and fill
// the issue slots where the others wait on their products and operand
// reads.  In the paired prefix loop those 4 run a loop of their own with no
// loads; elsewhere they still issue the staging loads -- the same addresses
// as the first 4, lines the caches already hold -- and skip only the
// conversions and LDS writes: with the loads behind a branch inside a loop,
// every wavefront ran one load sequence or another and the compiler waited
// for all loads in flight where the paths joined.  (Measured against 8 wavefronts, 32K prefix: NVFP4
// 4.60 -> 4.36 ms, INT4 4.91 -> 4.51 ms; INT4 220K prefix 30.2 -> 27.5 ms.)
// The paged kernels are held to 168 registers, with a few spills; the
// workspace variant (238 registers: its two-level output sums) keeps 8.
template <int SRC>
struct ExtCfg {
  static constexpr int WAVES = SRC == kExtWorkspace ? 8 : 12;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int ROWS = 16 * WAVES;
  static constexpr int WPE = WAVES / 4;
};

template <int D, int SRC>
__global__ __launch_bounds__(ExtCfg<SRC>::THREADS) __attribute__((amdgpu_waves_per_eu(ExtCfg<SRC>::WPE))) void extend_kernel(const ExtendParams p) {
  constexpr int kExtRows = ExtCfg<SRC>::ROWS;
  using Lds = ExtLds<D>;
  constexpr bool PAGED = SRC != kExtWorkspace;
  constexpr int KCH = D / 32, VT = D / 16;
  constexpr int KV16 = D / 128;      // 16-byte K vectors (staging passes) per thread and step
  extern __shared__ __attribute__((aligned(16))) uint8_t lds_mem[];
  lds_u8* const lds = (lds_u8*)lds_mem;

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane >> 4, n = lane & 15;
  // XCD-aware order: workgroups are dealt to the 8 XCDs round-robin in launch
  // order, so launch index w runs on XCD w mod 8.  Remapping w to the logical
  // (row block, KV head) gives each XCD one contiguous range of row blocks --
  // those resident together walk the same head's keys in step and share its
  // L2 -- instead of every head's keys passing through every XCD's L2.
  const int nwg = gridDim.x * gridDim.y, w = blockIdx.x + gridDim.x * blockIdx.y;
  const int per = nwg / 8, rem = nwg % 8, xcd = w % 8;
  const int lw = (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + w / 8;
  const int bx = lw % gridDim.x, g = lw / gridDim.x;
  const int G = p.group;
  const int64_t nrows = (int64_t)p.chunk_len * G;
  const int64_t row0 = (int64_t)bx * kExtRows;
  const int64_t Lk = (int64_t)p.prefix_len + p.chunk_len;

  // this lane's query row (column n of its wavefront's tile)
  const int64_t row = row0 + 16 * wave + n;
  const bool row_ok = row < nrows;
  const int irow = row_ok ? (int)(row / G) : p.chunk_len - 1;  // a padding row sees every key, q = 0
  const int h = g * G + (row_ok ? (int)(row % G) : 0);
  const int64_t lim = (int64_t)p.prefix_len + irow;            // last key the row sees

  // keys the workgroup needs: up to the last row's limit
  const int64_t last_row = min(row0 + kExtRows, nrows) - 1;
  const int64_t kmax = min(Lk - 1, (int64_t)p.prefix_len + last_row / G);
  // every row of the workgroup sees keys 0 .. lim_min: steps below it need no causal mask
  const int64_t lim_min = (int64_t)p.prefix_len + row0 / G;
  const int nsteps = (int)(kmax / kExtStep) + 1;

  // NVFP4 global scales, read once (a scalar load inside the loop would wait
  // on the LDS counter it shares)
  float gsf[2] = {1.0f, 1.0f};
  if (SRC == FMT_NVFP4) {
    gsf[0] = p.gs[0];
    gsf[1] = p.gs[1];
  }
  // Paged prefix: the steps whose 32 keys all lie in the cached prefix (every
  // row sees all of them: no mask) run in fp16, with p in fp16 (11 bits)
  // feeding a single PV MFMA.  NVFP4 codes are expanded as
  // (e2m1 * 2^8) * (E4M3 * 2^-8), exact, and the global scales, uniform over
  // these steps, go to the score (K) and, once after the last of them, to the
  // output accumulators (V).  INT4 codes are the integers q, exact, with the
  // token scales staged per token as on the bf16 steps; the value scale rides
  // on p, so the running max also bounds p * scale (below).  The steps from
  // the first one that reaches the chunk on take the bf16 path.
  constexpr bool F16P = PAGED;
  const int nsteps16 = F16P ? (int)min((int64_t)p.prefix_len / kExtStep, (int64_t)nsteps - 1) : 0;

  // the query row's MFMA operands: bf16 bits, or on the fp16 steps fp16 bits
  // of q * 2^kq, the power of two that puts the row's largest magnitude in
  // [2^14, 2^15) (every bf16 element within 2^31 of it is then exact)
  u32x4_t qw[KCH];
  auto load_q = [&]() {
    const uint16_t* qrow = p.q + (int64_t)irow * p.q_stride + (int64_t)h * D + 8 * j;
#pragma unroll
    for (int m = 0; m < KCH; m++) {
      u32x4_t raw = ld_global<u32x4_t>(qrow + 32 * m);
      if (!row_ok) raw = (u32x4_t){0u, 0u, 0u, 0u};
      qw[m] = raw;
    }
  };
  load_q();
  float ck = 1.0f;  // fp16 steps: gs_K * 2^-kq turns the MFMA sum into the score
  if (F16P && nsteps16 > 0) {
    float qmax = 0.0f;
#pragma unroll
    for (int m = 0; m < KCH; m++) {
      const uint32_t wq[4] = {qw[m].x, qw[m].y, qw[m].z, qw[m].w};
#pragma unroll
      for (int c = 0; c < 4; c++)
        qmax = fmaxf(qmax, fmaxf(__builtin_fabsf(as_f32(wq[c] << 16)), __builtin_fabsf(as_f32(wq[c] & 0xFFFF0000u))));
    }
    qmax = max_xor16_xor32(qmax);  // lanes n, n + 16, n + 32, n + 48 hold the row
    int qexp = 0;
    if (qmax > 0.0f) (void)frexpf(qmax, &qexp);  // qmax < 2^qexp
    const int kq = qmax > 0.0f ? 15 - qexp : 0;
#pragma unroll
    for (int m = 0; m < KCH; m++) {
      uint32_t wq[4] = {qw[m].x, qw[m].y, qw[m].z, qw[m].w};
#pragma unroll
      for (int c = 0; c < 4; c++)
        wq[c] = h2_as_u32((half2_t){(_Float16)ldexpf(as_f32(wq[c] << 16), kq),
                                    (_Float16)ldexpf(as_f32(wq[c] & 0xFFFF0000u), kq)});
      qw[m] = (u32x4_t){wq[0], wq[1], wq[2], wq[3]};
    }
    ck = (SRC == FMT_NVFP4 ? gsf[0] : 1.0f) * ldexpf(1.0f, -kq);
  }
  // scores stay unscaled (q.k, times the token's factor in the paged variant);
  // the running max is kept in the same units and p = 2^(s sm - m sm) is one
  // fma and one exp
  const float sm = p.sm_scale * kExtLog2e;
  const float slack_raw = kExtSlack / sm, inv_sm = 1.0f / sm;

  // ---- staging.  A quarter-wavefront writes 256 contiguous bytes of one
  // staged row per pass, which is conflict-free whatever the row's offset.
  // Workspace variant: pass v (< KV16) of thread t loads 16-byte segment kseg
  // of row krow0 + v * KRP (a wavefront reads whole rows).  Paged variant: 16
  // threads per row, one row per thread (one page lookup per row and step):
  // thread (krow0, kseg) takes the 8 elements from 8 kseg + v D/2 in pass v,
  // i.e. one 4-byte code word and (NVFP4) one E4M3 block scale per pass.
  // V rows are staged exactly like K rows.
  constexpr int KSEG = PAGED ? 16 : D / 8, KRP = kExtStagers / KSEG;
  const bool stager = wave < kExtStagers / 64;  // wave-uniform
  const int stid = tid % kExtStagers;  // wavefronts 8.. load what wavefronts 0.. load, then drop it
  const int krow0 = stid / KSEG, kseg = stid % KSEG;
  // bit position of this thread's NVFP4 block-scale byte (block kseg / 2 +
  // v D/32) in the aligned dword load_paged_row reads
  const int nv_sshift = 8 * ((kseg >> 1) & 3);
  // row and first element of pass v
  auto krow_of = [&](int v) { return PAGED ? krow0 : krow0 + v * KRP; };
  auto kel_of = [&](int v) { return PAGED ? 8 * kseg + (D / 2) * v : 8 * kseg; };
  const int64_t Lp = p.prefix_len;
  // bf16 rows: the workspace holds every token; the paged variant's rows are the chunk's
  const int64_t row_base = PAGED ? Lp : 0;
  // staged rows in flight: bf16 values, or for a paged prefix row per pass
  // its raw code word (reg[v].x) and scale word (reg[v].y), expanded in lstore
  u32x4_t kreg[KV16], vreg[KV16];
  // bf16 rows through buffer descriptors rebased per step (uniform, scalar
  // math); the record count ends at row Lk, so rows past the end read zeros,
  // and the lane parts of the offsets are loop-invariant
  const int kvo = (krow0 * (int)p.kv_stride + g * D + kel_of(0)) * 2;
  const int rowb = (int)p.kv_stride * 2;
  auto rows_rsrc = [&](const uint16_t* rows, int64_t t0) {
    const int64_t bytes = min((Lk - t0) * p.kv_stride * 2, (int64_t)0x7FFFFFF0);
    return __builtin_amdgcn_make_buffer_rsrc((void*)(rows + (t0 - row_base) * p.kv_stride), (short)0, (int)bytes,
                                             0x00020000);
  };
  // paged prefix: page-table slot and row of this thread's row (krow0) in the
  // step starting at token t0.  The step's first token sits in page t0 / P at
  // row t0 % P; a page holds at least 16 rows, so a token of the step is at
  // most two pages further.
  // Token indices of the prefix fit 31 bits, so the step's page is a
  // multiply-high by floor((2^32 - 1) / P), which is the quotient or one less,
  // and one correction (instead of a 64-bit division every step).
  const uint32_t psz = (uint32_t)p.page_size;
  const uint32_t pmagic = PAGED ? 0xFFFFFFFFu / psz : 0u;
  auto page_slot = [&](int64_t t0, int& off) -> int {
    const uint32_t t = (uint32_t)t0;
    uint32_t pi = __umulhi(t, pmagic);
    uint32_t o = t - pi * psz;
    if (o >= psz) { o -= psz; pi++; }
    o += (uint32_t)krow0;
    if (o >= psz) { o -= psz; pi++; }
    if (o >= psz) { o -= psz; pi++; }
    off = (int)o;
    return (int)pi;
  };
  // the page holding this thread's row of a step, read from the page table
  // one step before the step's codes are loaded, so the code loads never wait
  // for it.  A branch-free buffer load whose record count ends at the
  // prefix's last page: a slot past it reads 0 (page 0, whose rows then go
  // unused), so the load counter sees the same loads on every path and its
  // waits stay exact.
  const __amdgpu_buffer_rsrc_t pages_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)p.pages, (short)0, PAGED ? (int)min(4 * ((Lp + p.page_size - 1) / p.page_size), (int64_t)0x7FFFFFF0) : 0,
      0x00020000);
  auto page_id = [&](int step) -> int {
    if (!PAGED) return 0;
    const int64_t t0 = min((int64_t)step * kExtStep, (int64_t)0x7FFFFFC0);
    int off;
    return __builtin_amdgcn_raw_buffer_load_b32(pages_rsrc, 4 * page_slot(t0, off), 0, 0);
  };
  // a prefix row's staging registers, K (kv 0) or V (kv 1): per pass the
  // code word of the pass's 8 elements and the aligned dword holding their
  // E4M3 block scale (NVFP4; shifted by nv_sshift where used -- a narrower
  // load's zero extension would be an instruction on the loaded value, and
  // waiting for it a stall) or the row's fp32 scale (INT4), kept raw
  auto load_paged_row = [&](u32x4_t(&reg)[KV16], int kv, int64_t t0, int pid) {
    int off;
    (void)page_slot(t0, off);
    const uint8_t* sl = p.pool + ((int64_t)pid * p.num_kv_heads + g) * p.slab + kv * p.half;
    const uint8_t* cp = sl + (int64_t)off * (D / 2) + 4 * kseg;
    const uint8_t* sc = sl + p.scales_off;
#pragma unroll
    for (int v = 0; v < KV16; v++) {
      reg[v].x = ld_global<uint32_t>(cp + (D / 4) * v);
      if (SRC == FMT_NVFP4)
        reg[v].y = ld_global<uint32_t>(sc + (int64_t)off * (D / 16) + (((kseg >> 1) + (D / 32) * v) & ~3));
      else
        reg[v].y = ld_global<uint32_t>(sc + (int64_t)off * 4);
    }
  };
  // Steps whose rows all lie in the prefix: every 16-row half of such a step
  // lies in one page (pages hold a multiple of 16 rows and steps start at
  // multiples of 32), and the rows a wavefront stages are one half
  // (wavefronts w mod 8 < 4: rows 0..15), so the half's page, its slab and
  // the row offset are wave-uniform, scalar, and each lane adds a constant.
  const int hs = (wave & 7) >> 2;
  const int cvo = (krow0 & 15) * (D / 2) + 4 * kseg;  // lane's code bytes in its half's first row
  const int svo = SRC == FMT_NVFP4 ? (krow0 & 15) * (D / 16) + ((kseg >> 1) & ~3) : (krow0 & 15) * 4;
  auto half_slot = [&](int step, int& off) -> int {
    const uint32_t t = (uint32_t)min((int64_t)step * kExtStep, (int64_t)0x7FFFFFC0) + 16u * (uint32_t)hs;
    uint32_t pi = __umulhi(t, pmagic);
    uint32_t o = t - pi * psz;
    if (o >= psz) { o -= psz; pi++; }
    off = (int)o;
    return (int)pi;
  };
  // the page of this wavefront's half of a step, as page_id (the same value in every lane)
  auto page_id16 = [&](int step) -> int {
    int off;
    return __builtin_amdgcn_raw_buffer_load_b32(pages_rsrc, 4 * half_slot(step, off), 0, 0);
  };
  auto load_paged_half = [&](u32x4_t(&reg)[KV16], int kv, int step, int pid) {
    int off;
    (void)half_slot(step, off);
    const int spid = __builtin_amdgcn_readfirstlane(pid);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.pool + ((int64_t)spid * p.num_kv_heads + g) * p.slab), (short)0, (int)p.slab, 0x00020000);
    const int cso = kv * (int)p.half + off * (D / 2);
    const int sso = kv * (int)p.half + (int)p.scales_off + off * (SRC == FMT_NVFP4 ? D / 16 : 4);
#pragma unroll
    for (int v = 0; v < KV16; v++) {
      reg[v].x = __builtin_amdgcn_raw_buffer_load_b32(rs, cvo + (D / 4) * v, cso, 0);
      reg[v].y = __builtin_amdgcn_raw_buffer_load_b32(rs, svo + (SRC == FMT_NVFP4 ? (D / 32) * v : 0), sso, 0);
    }
  };
  // the loads of a step whose rows all lie in the prefix: no branch between
  // page and bf16 rows, so the loads land in their staging registers (a
  // register copy after a branch would wait for the load it copies)
  auto gload16 = [&](u32x4_t(&kr)[KV16], u32x4_t(&vr)[KV16], int step, int pid) {
    load_paged_half(kr, 0, step, pid);
    load_paged_half(vr, 1, step, pid);
  };
  // a bf16 row's staging registers (K: kv 0, V: kv 1)
  auto load_bf16_row = [&](u32x4_t(&reg)[KV16], int kv, int64_t t0) {
    const __amdgpu_buffer_rsrc_t rs = rows_rsrc(kv ? p.v : p.k, t0);
#pragma unroll
    for (int v = 0; v < KV16; v++)
      reg[v] = __builtin_amdgcn_raw_buffer_load_b128(rs, kvo + (PAGED ? D * v : v * KRP * rowb), 0, 0);
  };
  auto gload = [&](int step, int pid) {
    const int64_t t0 = (int64_t)step * kExtStep;
    // one row's staging registers: K (kv 0) or V (kv 1)
    auto rows = [&](u32x4_t(&reg)[KV16], int kv) {
      if (PAGED && t0 + krow0 < Lp)
        load_paged_row(reg, kv, t0, pid);
      else
        load_bf16_row(reg, kv, t0);
    };
    rows(kreg, 0);
    rows(vreg, 1);
  };
  // the loads of a step whose rows all lie in the chunk (paged variant): bf16
  // rows only, no branch (as gload16 for the prefix)
  auto gloadc = [&](int step) {
    const int64_t t0 = (int64_t)step * kExtStep;
    load_bf16_row(kreg, 0, t0);
    load_bf16_row(vreg, 1, t0);
  };
  // bf16 pairs of 8 codes (element 0 low): NVFP4 e2m1 * block scale, exact;
  // INT4 the integers q, exact
  auto expand8 = [&](uint32_t w, float s, uint32_t out[4]) {
#pragma unroll
    for (int e = 0; e < 4; e++) {
      float2_t x;
      if (SRC == FMT_NVFP4) {
        switch (e) {
          case 0: x = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0); break;
          case 1: x = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1); break;
          case 2: x = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2); break;
          default: x = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3); break;
        }
        x[0] *= s;
        x[1] *= s;
      } else {
        x[0] = (float)((int)(w << (28 - 8 * e)) >> 28);
        x[1] = (float)((int)(w << (24 - 8 * e)) >> 28);
      }
      out[e] = bf16x2_rne(x);
    }
  };
  auto lstore = [&](int buf, int64_t t0) {
    if (!stager) return;
    lds_u8* base = lds + buf * Lds::BUF;
    lds_f32* fac = (lds_f32*)(base + Lds::KB + Lds::VB);  // [K factors][V factors], one per token
    auto stage = [&](u32x4_t(&reg)[KV16], int kv) {
      if (PAGED) {
        const bool pg = t0 + krow0 < Lp;
        const uint32_t rs = reg[0].y;  // INT4 row scale, read before the expansion overwrites it
        if (pg) {
#pragma unroll
          for (int v = 0; v < KV16; v++) {
            uint32_t o[4];
            expand8(reg[v].x, SRC == FMT_NVFP4 ? e4m3_decode((reg[v].y >> nv_sshift) & 0xFFu) : 1.0f, o);
            reg[v] = (u32x4_t){o[0], o[1], o[2], o[3]};
          }
        }
        if (kseg == 0) fac[kv * kExtStep + krow0] = pg ? (SRC == FMT_NVFP4 ? gsf[kv] : as_f32(rs)) : 1.0f;
      }
      lds_u8* rbase = base + kv * Lds::KB;
#pragma unroll
      for (int v = 0; v < KV16; v++)
        *(lds_u32x4*)(rbase + (krow_of(v) * Lds::KPD + kel_of(v) / 2) * 4) = reg[v];
    };
    stage(kreg, 0);
    stage(vreg, 1);
  };
  // fp16 staging of a prefix step (every row of it in the prefix).  NVFP4: per
  // code word, four conversions at a 2^8 scale and four packed multiplies by
  // the block scale times 2^-8, exact (e2m1 * E4M3 has at most 6 significant
  // bits and lies in [2^-10, 2688]).  INT4: byte k of the word and of the word
  // shifted by 4 side by side put nibbles 2k and 2k + 1 in the low bits of the
  // two halves, which land in the mantissa of 1024 with the sign bit flipped
  // (q + 8), less 1032: q exactly, three instructions per pair; the token's
  // scale is staged as on the bf16 steps.
  auto lstore16 = [&](u32x4_t(&kr)[KV16], u32x4_t(&vr)[KV16], int buf) {
    if (!stager) return;
    lds_u8* base = lds + buf * Lds::BUF;
    lds_f32* fac = (lds_f32*)(base + Lds::KB + Lds::VB);
    auto stage = [&](u32x4_t(&reg)[KV16], int kv) {
      const uint32_t rs = reg[0].y;  // INT4 row scale
#pragma unroll
      for (int v = 0; v < KV16; v++) {
        const uint32_t cw = reg[v].x;
        if constexpr (SRC == FMT_NVFP4) {
          const uint32_t hb = e4m3_to_h_x2m8(reg[v].y >> nv_sshift);
          const half2_t s2 = u32_as_h2(hb | (hb << 16));
          reg[v] = (u32x4_t){h2_as_u32(e2m1x2_to_h2_x256<0>(cw) * s2), h2_as_u32(e2m1x2_to_h2_x256<1>(cw) * s2),
                             h2_as_u32(e2m1x2_to_h2_x256<2>(cw) * s2), h2_as_u32(e2m1x2_to_h2_x256<3>(cw) * s2)};
        } else {
          const uint32_t w = cw, w4 = w >> 4;
          uint32_t o[4];
#pragma unroll
          for (int k = 0; k < 4; k++) {
            const uint32_t t = (byte_perm(w4, w, (uint32_t)k | 0x0C00u | ((uint32_t)(4 + k) << 16) | 0x0C000000u) &
                                0x000F000Fu) ^ 0x64086408u;
            o[k] = h2_as_u32(u32_as_h2(t) - (half2_t){(_Float16)1032.0f, (_Float16)1032.0f});
          }
          reg[v] = (u32x4_t){o[0], o[1], o[2], o[3]};
        }
      }
      if (SRC == FMT_INT4 && kseg == 0) fac[kv * kExtStep + krow0] = as_f32(rs);
      lds_u8* rbase = base + kv * Lds::KB;
#pragma unroll
      for (int v = 0; v < KV16; v++)
        *(lds_u32x4*)(rbase + (krow_of(v) * Lds::KPD + kel_of(v) / 2) * 4) = reg[v];
    };
    stage(kr, 0);
    stage(vr, 1);
  };

  float4_t oacc[VT];
#pragma unroll
  for (int t = 0; t < VT; t++) oacc[t] = (float4_t){0.0f, 0.0f, 0.0f, 0.0f};
  float m_run = -__builtin_inff(), l_run = 0.0f;
  // Two-level accumulation.  The MFMA accumulation aligns each product to
  // the accumulator's exponent and keeps only about 3 bits below its ulp
  // (measured on gfx950: with C = 1.0, 32 products of 2^-27 add nothing), and
  // an fp32 sum of many small terms into a large one loses every term below
  // half its ulp; over the tens of thousands of steps of a long prefix both
  // drop the small late contributions with a bias.  So the running sums
  // restart from zero every kExtFlush steps and are added into totals on VALU
  // (round to nearest): l_run into l_tot always, oacc into otot in the
  // workspace variant (the paged variant has no registers to spare for it).
  constexpr bool TWO_LEVEL = !PAGED;
  float4_t otot[TWO_LEVEL ? VT : 1];
#pragma unroll
  for (int t = 0; t < (TWO_LEVEL ? VT : 1); t++) otot[t] = (float4_t){0.0f, 0.0f, 0.0f, 0.0f};
  float l_tot = 0.0f;
  auto flush = [&]() {
    l_tot += l_run;
    l_run = 0.0f;
    if constexpr (TWO_LEVEL) {
#pragma unroll
      for (int t = 0; t < VT; t++) {
        otot[t] += oacc[t];
        oacc[t] = (float4_t){0.0f, 0.0f, 0.0f, 0.0f};
      }
    }
  };

  // one step: F16 (a std::bool_constant) selects the fp16 prefix form
  auto compute = [&](auto f16_tag, int buf, int64_t t0) {
    constexpr bool F16 = decltype(f16_tag)::value;
    const lds_u8* kb = lds + buf * Lds::BUF;
    const lds_u8* vrows = kb + Lds::KB;
    // the two 16-token halves are independent accumulation chains: their
    // products alternate, so neither waits on its own previous product
    float4_t sacc[2];
    sacc[0] = sacc[1] = (float4_t){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int m = 0; m < KCH; m++) {
#pragma unroll
      for (int hh = 0; hh < 2; hh++) {
        const u32x4_t a = *(const lds_u32x4*)(kb + (16 * hh + n) * Lds::KPD * 4 + 16 * j + 64 * m);
        if constexpr (F16)
          sacc[hh] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a),
                                                            __builtin_bit_cast(half8_t, qw[m]), sacc[hh], 0, 0, 0);
        else
          sacc[hh] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                             __builtin_bit_cast(bf16x8_t, qw[m]), sacc[hh], 0, 0, 0);
      }
    }
    // operand reads four products ahead of the products that use them
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < 2 * KCH - 4; i++) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    float s[8], vf[8], cand[8];
    const lds_f32* kfac = (const lds_f32*)(kb + Lds::KB + Lds::VB);
    const lds_f32* vfac = kfac + kExtStep;
    float cmax = -__builtin_inff();
    // fp16 steps lie below every row's causal limit
    const bool masked = !F16 && t0 + kExtStep - 1 > lim_min;  // workgroup-uniform
    const int last = (int)min(lim - t0, (int64_t)kExtStep);  // last visible token of the step, in step units
#pragma unroll
    for (int e = 0; e < 8; e++) {
      const int tok = 16 * (e / 4) + 4 * j + (e % 4);
      float x = sacc[e / 4][e % 4];
      if (F16) x *= ck;
      if (SRC == FMT_INT4 || (PAGED && !F16)) {
        x *= kfac[tok];
        vf[e] = vfac[tok];
      }
      s[e] = x;
      // INT4 fp16 steps: the running max also bounds p * (value scale), so
      // the product p' stays below 2^slack in fp16; the scale's binary
      // exponent (scale < 2^e) is the bound, clamped so that tiny scales
      // cannot push p out of fp32 range
      if (F16 && SRC == FMT_INT4) cand[e] = x + (float)max(__builtin_amdgcn_frexp_expf(vf[e]), -64) * inv_sm;
    }
    // only steps that reach a row's causal limit need the mask (a
    // workgroup-uniform test, so the others skip it)
    if (masked) {
#pragma unroll
      for (int e = 0; e < 8; e++)
        if (16 * (e / 4) + 4 * j + (e % 4) > last) s[e] = -__builtin_inff();
    }
#pragma unroll
    for (int e = 0; e < 8; e++) cmax = fmaxf(cmax, F16 && SRC == FMT_INT4 ? cand[e] : s[e]);
    // a row's max can only pass m_run + slack where one of its lanes' own
    // maxima does, so the wave-wide test needs no cross-lane reduction; the
    // row max (over the row's 4 lanes) is formed only when some row moves
    if (__builtin_amdgcn_ballot_w64(cmax > m_run + slack_raw) != 0) {
      cmax = max_xor16_xor32(cmax);
      const float m_new = cmax > m_run + slack_raw ? cmax : m_run;
      const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * sm);
      m_run = m_new;
      l_run *= alpha;
      l_tot *= alpha;
#pragma unroll
      for (int t = 0; t < VT; t++) oacc[t] *= alpha;
      if constexpr (TWO_LEVEL) {
#pragma unroll
        for (int t = 0; t < VT; t++) otot[t] *= alpha;
      }
    }
    const float msm = m_run * sm;
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[e], sm, -msm));
      float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[e + 1], sm, -msm));
      l_run += p0 + p1;
      if constexpr (F16) {
        if (SRC == FMT_INT4) {  // the token's value scale rides on its probability
          p0 *= vf[e];
          p1 *= vf[e + 1];
        }
        hi[e / 2] = h2_as_u32((half2_t){(_Float16)p0, (_Float16)p1});
        lo[e / 2] = 0u;
      } else {
        if (PAGED) {  // the value factor of each token rides on its probability
          p0 *= vf[e];
          p1 *= vf[e + 1];
        }
        const uint32_t hw = bf16x2_rne((float2_t){p0, p1});
        const float h0 = as_f32(hw << 16), h1 = as_f32(hw & 0xFFFF0000u);
        hi[e / 2] = hw;
        lo[e / 2] = bf16x2_rne((float2_t){p0 - h0, p1 - h1});
      }
    }
    const u32x4_t phi = (u32x4_t){hi[0], hi[1], hi[2], hi[3]};
    const u32x4_t plo = (u32x4_t){lo[0], lo[1], lo[2], lo[3]};
    // PV operand of tile t for lane (j, n): channel 16t + n of tokens 4j..4j+3
    // and 16+4j..16+4j+3 (the order of P's k index), by two transposing reads:
    // lane (j, n) names channels 16t + 4(n%4) .. +3 of token row 4j + n/4
    // (then 16 + 4j + n/4) and receives channel 16t + n of the group's 4 rows
    const lds_u8* vop = vrows + ((4 * j + (n >> 2)) * Lds::KPD + 2 * (n & 3)) * 4;
#pragma unroll
    for (int t = 0; t < VT; t++) {
      const v4i16_t lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_ptr)(vop + 32 * t));
      const v4i16_t hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_ptr)(vop + 32 * t + 16 * Lds::KPD * 4));
      const u32x4_t a = (u32x4_t){__builtin_bit_cast(u32x2_t, lo4).x, __builtin_bit_cast(u32x2_t, lo4).y,
                                  __builtin_bit_cast(u32x2_t, hi4).x, __builtin_bit_cast(u32x2_t, hi4).y};
      if constexpr (F16) {
        oacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a), __builtin_bit_cast(half8_t, phi),
                                                         oacc[t], 0, 0, 0);
      } else {
        const bf16x8_t ab = __builtin_bit_cast(bf16x8_t, a);
        oacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ab, __builtin_bit_cast(bf16x8_t, phi), oacc[t], 0, 0, 0);
        oacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ab, __builtin_bit_cast(bf16x8_t, plo), oacc[t], 0, 0, 0);
      }
    }
  };

  int pid = page_id(0);
  gload(0, pid);
  if (F16P && nsteps16 > 0)
    lstore16(kreg, vreg, 0);
  else
    lstore(0, 0);
  pid = page_id(1);
  if (nsteps > 1) gload(1, pid);
  pid = page_id(2);
  // the page entry of step 3's half, for the second staging set of the paired prefix loop below
  const int pid3 = PAGED ? page_id16(3) : 0;
  __syncthreads();
  // stage step st + 1 (in its own form) and issue the loads of step st + 2
  auto advance = [&](int st) {
    if (st + 1 < nsteps) {
      if (F16P && st + 1 < nsteps16)
        lstore16(kreg, vreg, (st + 1) & 3);
      else
        lstore((st + 1) & 3, (int64_t)(st + 1) * kExtStep);
      if (st + 2 < nsteps) {
        gload(st + 2, pid);
        pid = page_id(st + 3);
      }
    }
    __syncthreads();
  };
  // Prefix steps, two per barrier: steps st and st + 1 are computed from
  // buffers st and st + 1 (mod 4) while steps st + 2 and st + 3 are staged
  // into the other two, from two staging sets (kreg, vreg; kreg2, vreg2)
  // whose loads -- steps st + 4 and st + 5 -- are issued right after, so a
  // set's loads have a pair of steps to land.  Each set's page entries are
  // fetched a pair of steps ahead (pid_a, pid_b), so that waiting for them
  // never waits for the other set's loads (the load counter is in order).
  u32x4_t kreg2[KV16], vreg2[KV16];
  int st = 0;
  if constexpr (F16P) {
    if (nsteps16 > 6) {
      // entering: buffer 0 holds step 0, the first set the loads of step 1.
      // The loads leave in the loop's own order -- a set's 8 loads, then
      // the page entry it uses next, then the other set's -- so that the
      // compiler's wait counts, which must hold for the first iteration as
      // for the others, wait for the entry alone and not for the other
      // set's loads as well (the scheduling barriers keep the order).
      // Wavefronts 8.. stage nothing and run a loop of their own without the
      // loads: with no staging registers live through its products, the
      // compiler keeps four key-operand reads in flight there instead of one.
      // Their staging registers hold constants on entry, so no loaded value
      // has to survive their loop; the two loops meet once, after it.
      if (stager) {
        lstore16(kreg, vreg, 1);
        gload16(kreg, vreg, 2, pid);
        int pid_a = page_id16(4);
        __builtin_amdgcn_sched_barrier(0);
        gload16(kreg2, vreg2, 3, pid3);
        int pid_b = page_id16(5);
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
        // INT4: the two staging wavefronts of a SIMD (w and w + 4) take the
        // pair in opposite orders -- stage then compute, compute then stage --
        // so one's conversions overlap the other's products instead of both
        // queuing for the matrix core at once.  NVFP4, whose compute-only
        // wavefronts fill the matrix core while both stage: stage first
        // (measured against the opposite orders in one run: NVFP4 4.10 ->
        // 4.00 ms at 32K and 26.4 -> 25.8 ms at 256K; INT4 4.14 -> 4.49 ms
        // at 32K).  Every order computes the same steps from the same buffers.
        const bool stage_first = SRC == FMT_NVFP4 || wave >= 4;
        auto stage_pair = [&](int st) {
          lstore16(kreg, vreg, (st + 2) & 3);
          gload16(kreg, vreg, st + 4, pid_a);
          pid_a = page_id16(st + 6);
          lstore16(kreg2, vreg2, (st + 3) & 3);
          gload16(kreg2, vreg2, st + 5, pid_b);
          pid_b = page_id16(st + 7);
        };
        for (; st + 5 < nsteps16; st += 2) {
          if (stage_first) stage_pair(st);
          compute(std::true_type{}, st & 3, (int64_t)st * kExtStep);
          compute(std::true_type{}, (st + 1) & 3, (int64_t)(st + 1) * kExtStep);
          if ((st + 2) % kExtFlush == 0) flush();  // st is even and kExtFlush a multiple of 2
          if (!stage_first) stage_pair(st);
          __syncthreads();
        }
      } else {
#pragma unroll
        for (int v = 0; v < KV16; v++) kreg[v] = vreg[v] = (u32x4_t){0u, 0u, 0u, 0u};
        __syncthreads();
        for (; st + 5 < nsteps16; st += 2) {
          compute(std::true_type{}, st & 3, (int64_t)st * kExtStep);
          compute(std::true_type{}, (st + 1) & 3, (int64_t)(st + 1) * kExtStep);
          if ((st + 2) % kExtFlush == 0) flush();
          __syncthreads();
        }
      }
      // back to one set: step st is computed here, step st + 1 is staged and
      // the first set holds the loads of step st + 2 (the second set's step
      // st + 3 is dropped and loaded again)
      compute(std::true_type{}, st & 3, (int64_t)st * kExtStep);
      if ((st + 1) % kExtFlush == 0) flush();
      st++;
      pid = page_id(st + 2);
    }
    for (; st < nsteps16; st++) {
      compute(std::true_type{}, st & 3, (int64_t)st * kExtStep);
      if ((st + 1) % kExtFlush == 0) flush();
      advance(st);
    }
    if (nsteps16 > 0) {
      // on to bf16: the query's bf16 operands again, and (NVFP4) the value
      // global scale of the prefix steps' sum applied once
      load_q();
      if (SRC == FMT_NVFP4) {
#pragma unroll
        for (int t = 0; t < VT; t++) oacc[t] *= gsf[1];
      }
    }
  }
  // paged variant: from the step whose prefetch target lies wholly in the
  // chunk on, the loads are gloadc's, issued on every step but the last two
  // (a conditional load would again need a register merge)
  const int st_chunk = PAGED ? (int)((Lp + kExtStep - 1) / kExtStep) : 0;  // first step with no prefix row
  for (; st < nsteps && (!PAGED || st + 2 < st_chunk); st++) {
    compute(std::false_type{}, st & 3, (int64_t)st * kExtStep);
    if ((st + 1) % kExtFlush == 0) flush();
    advance(st);
  }
  if constexpr (PAGED) {
    for (; st + 2 < nsteps; st++) {
      compute(std::false_type{}, st & 3, (int64_t)st * kExtStep);
      if ((st + 1) % kExtFlush == 0) flush();
      lstore((st + 1) & 3, (int64_t)(st + 1) * kExtStep);
      gloadc(st + 2);
      __syncthreads();
    }
    for (; st < nsteps; st++) {
      compute(std::false_type{}, st & 3, (int64_t)st * kExtStep);
      if ((st + 1) % kExtFlush == 0) flush();
      advance(st);
    }
  }

  // ---- epilogue: each lane column is one query row
  if constexpr (TWO_LEVEL) {
#pragma unroll
    for (int t = 0; t < VT; t++) oacc[t] += otot[t];
  }
  l_run += l_tot;
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  if (!row_ok) return;
  const float inv = l_run > 0.0f ? 1.0f / l_run : 0.0f;
  const int64_t obase = (int64_t)irow * p.out_stride + (int64_t)h * D + 4 * j;
#pragma unroll
  for (int t = 0; t < VT; t++) {
    const float o0 = oacc[t][0] * inv, o1 = oacc[t][1] * inv, o2 = oacc[t][2] * inv, o3 = oacc[t][3] * inv;
    if (p.out_bf16) {
      *(u32x2_t*)((uint16_t*)p.out + obase + 16 * t) =
          (u32x2_t){bf16x2_rne((float2_t){o0, o1}), bf16x2_rne((float2_t){o2, o3})};
    } else {
      *(float4*)((float*)p.out + obase + 16 * t) = make_float4(o0, o1, o2, o3);
    }
  }
  if (p.lse != nullptr && j == 0)
    p.lse[(int64_t)irow * p.lse_stride + h] = l_run > 0.0f ? (m_run * sm + log2f(l_run)) * kExtLn2 : -__builtin_inff();
}

// The four staging buffers (140 KB at head dim 256) are above HIP's default
// 64 KB dynamic-LDS limit per workgroup (gfx950 has 160 KB per CU), so each
// instantiation raises its limit -- once per device, on its first launch
// there, not on every launch (a host call that a captured graph would
// otherwise repeat).  A failure is kept and returned by every later launch.
constexpr int kExtMaxDevices = 64;

template <int D, int SRC>
static hipError_t extend_lds_limit() {
  static std::once_flag once[kExtMaxDevices];
  static hipError_t result[kExtMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kExtMaxDevices) {
    (void)hipGetLastError();
    return hipFuncSetAttribute((const void*)extend_kernel<D, SRC>, hipFuncAttributeMaxDynamicSharedMemorySize,
                               ExtLds<D>::TOTAL);
  }
  std::call_once(once[dev], [dev] {
    result[dev] = hipFuncSetAttribute((const void*)extend_kernel<D, SRC>,
                                      hipFuncAttributeMaxDynamicSharedMemorySize, ExtLds<D>::TOTAL);
  });
  return result[dev];
}

template <int D, int SRC>
static hipError_t launch_extend_t(const ExtendParams& p, hipStream_t stream) {
  const int64_t rows = (int64_t)p.chunk_len * p.group;
  constexpr int R = ExtCfg<SRC>::ROWS;
  const dim3 grid((unsigned)((rows + R - 1) / R), (unsigned)p.num_kv_heads), block(ExtCfg<SRC>::THREADS);
  const hipError_t e = extend_lds_limit<D, SRC>();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((extend_kernel<D, SRC>), grid, block, ExtLds<D>::TOTAL, stream, p);
  return hipGetLastError();
}

hipError_t launch_extend(const ExtendParams& p, int head_dim, int src_fmt, hipStream_t stream) {
  if (head_dim == 256) {
    if (src_fmt == FMT_NVFP4) return launch_extend_t<256, FMT_NVFP4>(p, stream);
    if (src_fmt == FMT_INT4) return launch_extend_t<256, FMT_INT4>(p, stream);
    return launch_extend_t<256, kExtWorkspace>(p, stream);
  }
  if (src_fmt == FMT_NVFP4) return launch_extend_t<128, FMT_NVFP4>(p, stream);
  if (src_fmt == FMT_INT4) return launch_extend_t<128, FMT_INT4>(p, stream);
  return launch_extend_t<128, kExtWorkspace>(p, stream);
}

}  // namespace kvq
