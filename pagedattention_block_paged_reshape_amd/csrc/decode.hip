// Paged decode attention on gfx950: the decode launch and its C entry points.
// The kernels and their design are in decode_core.h.
#include <algorithm>
#include <mutex>

#include "decode_core.h"

// Partials of pa_paged_attention_decode_noalloc, for callers that cannot
// allocate: a device array of the library's code object, one per GPU,
// created when the code is loaded on that GPU and held until the process
// ends.  Host code never uses this name as an address (on the host it is a
// stand-in, not device memory); it uses the address hipGetSymbolAddress
// gives for each device.
static __device__ __align__(256) unsigned char scratch[PA_DECODE_SCRATCH_BYTES];

namespace pa {

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device, once looked up
}  // namespace

// The scratch array's device address on the current device (looked up on
// the first call for that device, with it current).
static pa_status scratch_on_current_device(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return PA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return PA_ERR_INVALID;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return PA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return PA_OK;
}

// The kernels of one (head_dim, KEEP, FP8) choice.
struct DecodeKernels {
  void (*worklist)(DecodeArgs, const int32_t*, int32_t, int32_t);
  void (*grid)(DecodeArgs);
};

template <int D, bool KEEP, bool FP8>
static DecodeKernels kernels_of() {
  return {&decode_worklist_kernel<D, KEEP, FP8>, &decode_partition_kernel<D, KEEP, FP8>};
}

static DecodeKernels pick_kernels(int D, bool keep, bool fp8) {
  if (D == 128) {
    if (fp8) return keep ? kernels_of<128, true, true>() : kernels_of<128, false, true>();
    return keep ? kernels_of<128, true, false>() : kernels_of<128, false, false>();
  }
  if (fp8) return keep ? kernels_of<64, true, true>() : kernels_of<64, false, true>();
  return keep ? kernels_of<64, true, false>() : kernels_of<64, false, false>();
}

// Resident workgroups of the work-list kernel on the current device (cached
// per kernel and G; the dynamic LDS depends on G).
static int worklist_resident_wgs(int D, bool keep, bool fp8, int G, size_t lds) {
  static int per_cu[2][2][2][17];
  static int cus = 0;
  int& slot = per_cu[D == 128 ? 1 : 0][keep ? 1 : 0][fp8 ? 1 : 0][G];
  if (slot == 0) {
    int n = 0;
    const void* fn = reinterpret_cast<const void*>(pick_kernels(D, keep, fp8).worklist);
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, kDecodeThreads, lds) != hipSuccess || n < 1)
      n = 1;
    slot = n;
  }
  if (cus == 0) {
    int dev = 0, c = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        c > 0)
      cus = c;
    else
      cus = 1;
  }
  return slot * cus;
}

static pa_status decode_launch(pa_half* out, const pa_half* q, const PoolArgs& kv,
                               const int32_t* tables, int32_t max_blocks,
                               const int32_t* seq_lens, int32_t batch, int32_t num_q_heads,
                               float scale, int32_t partition_size, int32_t max_seq_len,
                               const int32_t* work_items, int32_t n_items, void* workspace,
                               uint64_t workspace_bytes, uint32_t flags, void* stream) {
  DecodeArgs a;
  const pa_status st = decode_prepare(out, q, kv, tables, max_blocks, seq_lens, batch,
                                      num_q_heads, scale, partition_size, max_seq_len,
                                      work_items, n_items, workspace, workspace_bytes, flags, a);
  if (st != PA_OK || batch == 0) return st;
  const bool keep = (flags & PA_DECODE_KEEP_KV) != 0;
  const bool worklist = work_items != nullptr;
  const int D = kv.head_dim;
  const int G = a.G;
  const int p_max = a.p_max;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const DecodeKernels kn = pick_kernels(D, keep, kv.fp8);
  if (worklist) {
    if (n_items > 0) {
      // result ring: as many unit slots as fit in ~16 KiB (at least 2)
      const size_t ring_slot = walk_ring_slot_bytes(G, D);
      const int ring = static_cast<int>(std::max<size_t>(2, kResultRingBytes / ring_slot));
      const size_t lds = walk_merge_bytes(G, D) + static_cast<size_t>(ring) * ring_slot;
      int wph = worklist_resident_wgs(D, keep, kv.fp8, G, lds) / kv.num_kv_heads;
      if (wph < 1) wph = 1;
      if (wph > n_items) wph = n_items;
      if (wph > 65535) wph = 65535;
      const dim3 grid(static_cast<uint32_t>(kv.num_kv_heads), static_cast<uint32_t>(wph));
      kn.worklist<<<grid, dim3(kDecodeThreads), lds, s>>>(a, work_items, n_items, ring);
    }
  } else {
    const size_t lds = static_cast<size_t>(kDecodeWaves) * G * (D + 4) * sizeof(float);
    const dim3 grid(static_cast<uint32_t>(kv.num_kv_heads), static_cast<uint32_t>(batch),
                    static_cast<uint32_t>(p_max));
    kn.grid<<<grid, dim3(kDecodeThreads), lds, s>>>(a);
  }
  if (hipGetLastError() != hipSuccess) return PA_ERR_HIP;
  if (p_max > 1) {
    const dim3 rgrid(static_cast<uint32_t>(kv.num_kv_heads), static_cast<uint32_t>(batch));
    if (D == 128)
      decode_reduce_kernel<128><<<rgrid, dim3(reduce_waves(p_max) * kWave),
                                 reduce_lds(p_max, a.G, 128), s>>>(a);
    else
      decode_reduce_kernel<64><<<rgrid, dim3(reduce_waves(p_max) * kWave),
                                 reduce_lds(p_max, a.G, 64), s>>>(a);
  }
  return launch_status();
}

}  // namespace pa

using namespace pa;

extern "C" uint64_t pa_decode_workspace_bytes(int32_t batch, int32_t num_q_heads,
                                              int32_t head_dim, int32_t max_seq_len,
                                              int32_t partition_size) {
  if (batch <= 0 || num_q_heads <= 0 || head_dim <= 0 || max_seq_len < 0 || partition_size <= 0)
    return 0;
  const uint64_t parts = max_seq_len == 0
                             ? 1
                             : (static_cast<uint64_t>(max_seq_len) + partition_size - 1) /
                                   partition_size;
  // fp16 normalised partial outputs, then fp32 running max and sum
  return parts > 1 ? static_cast<uint64_t>(batch) * num_q_heads * parts * (head_dim * 2 + 8) : 0;
}

extern "C" pa_status pa_paged_attention_decode(pa_half* out, const pa_half* q, pa_kv_view kv,
                                               const int32_t* tables, int32_t max_blocks,
                                               const int32_t* seq_lens, int32_t batch,
                                               int32_t num_q_heads, float scale,
                                               int32_t partition_size, int32_t max_seq_len,
                                               const int32_t* work_items, int32_t n_items,
                                               void* workspace, uint64_t workspace_bytes,
                                               uint32_t flags, void* stream) {
  const PoolArgs pk{kv.k_pool, kv.v_pool, kv.num_blocks, kv.block_size, kv.num_kv_heads,
                    kv.head_dim, false, 1.0f, 1.0f};
  return decode_launch(out, q, pk, tables, max_blocks, seq_lens, batch, num_q_heads, scale,
                       partition_size, max_seq_len, work_items, n_items, workspace,
                       workspace_bytes, flags, stream);
}

extern "C" pa_status pa_paged_attention_decode_fp8(
    pa_half* out, const pa_half* q, pa_kv_view_fp8 kv, const int32_t* tables, int32_t max_blocks,
    const int32_t* seq_lens, int32_t batch, int32_t num_q_heads, float scale,
    int32_t partition_size, int32_t max_seq_len, const int32_t* work_items, int32_t n_items,
    void* workspace, uint64_t workspace_bytes, uint32_t flags, void* stream) {
  const PoolArgs pk{kv.k_pool, kv.v_pool, kv.num_blocks, kv.block_size, kv.num_kv_heads,
                    kv.head_dim, true, kv.k_scale, kv.v_scale};
  return decode_launch(out, q, pk, tables, max_blocks, seq_lens, batch, num_q_heads, scale,
                       partition_size, max_seq_len, work_items, n_items, workspace,
                       workspace_bytes, flags, stream);
}

extern "C" pa_status pa_paged_attention_decode_noalloc(
    pa_half* out, const pa_half* q, pa_kv_view kv, const int32_t* tables, int32_t max_blocks,
    const int32_t* seq_lens, int32_t batch, int32_t num_q_heads, float scale,
    int32_t partition_size, int32_t max_seq_len, const int32_t* work_items, int32_t n_items,
    uint32_t flags, void* stream) {
  // the partials must fit the scratch array: refused before anything else
  const uint64_t need = pa_decode_workspace_bytes(batch, num_q_heads, kv.head_dim, max_seq_len,
                                                  partition_size);
  if (need > PA_DECODE_SCRATCH_BYTES) return PA_ERR_CAPACITY;
  // the launch goes to the stream's device, which must be the current one
  // (the scratch address is per device)
  if (stream != nullptr) {
    int cur = 0;
    hipDevice_t sdev = 0;
    if (hipGetDevice(&cur) != hipSuccess ||
        hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev) != hipSuccess)
      return PA_ERR_HIP;
    if (sdev != cur) return PA_ERR_INVALID;
  }
  void* ws = nullptr;
  if (need > 0) {
    const pa_status st = scratch_on_current_device(&ws);
    if (st != PA_OK) return st;
  }
  const PoolArgs pk{kv.k_pool, kv.v_pool, kv.num_blocks, kv.block_size, kv.num_kv_heads,
                    kv.head_dim, false, 1.0f, 1.0f};
  return decode_launch(out, q, pk, tables, max_blocks, seq_lens, batch, num_q_heads, scale,
                       partition_size, max_seq_len, work_items, n_items, ws, need, flags, stream);
}
