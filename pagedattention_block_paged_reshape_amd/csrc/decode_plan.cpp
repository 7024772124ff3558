// Host planner for the work-list form of paged decode: the (request,
// partition) units of one decode step, largest first.  Pure C++17, no GPU
// runtime.
//
// Each request of length L is cut into ceil(ceil(L/16) / part_blocks)
// partitions of part_blocks 16-token blocks (the last one may be shorter);
// a request of length 0 contributes one empty unit so that its output is
// still written (as zeros).  Units are ordered by block count, descending,
// ties in (request, partition) order, so that the units the GPU starts last
// are the short ones.
#include <climits>
#include <cstddef>
#include <cstdint>
#include <vector>

#include "pa.h"

extern "C" int32_t pa_decode_work_items(const int32_t* seq_lens, int32_t batch,
                                        int32_t partition_size, int32_t* items, int32_t cap) {
  if (batch < 0 || batch > 65535 || cap < 0) return -PA_ERR_INVALID;
  if (batch > 0 && seq_lens == nullptr) return -PA_ERR_INVALID;
  if (partition_size <= 0 || partition_size % PA_BLOCK_SIZE != 0) return -PA_ERR_INVALID;
  const int64_t part_blocks = partition_size / PA_BLOCK_SIZE;
  // bucket units by size (blocks), keeping (request, partition) order inside
  std::vector<std::vector<int32_t>> by_size(static_cast<size_t>(part_blocks) + 1);
  int64_t n = 0;
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t L = seq_lens[b];
    if (L < 0) return -PA_ERR_INVALID;
    if (L == 0) {
      by_size[0].push_back(static_cast<int32_t>(static_cast<uint32_t>(b) << 16));
      ++n;
      continue;
    }
    const int64_t nb = (L + PA_BLOCK_SIZE - 1) / PA_BLOCK_SIZE;
    const int64_t parts = (nb + part_blocks - 1) / part_blocks;
    if (parts > 65535) return -PA_ERR_INVALID;
    for (int64_t p = 0; p < parts; ++p) {
      const int64_t size = nb - p * part_blocks < part_blocks ? nb - p * part_blocks : part_blocks;
      by_size[static_cast<size_t>(size)].push_back(
          static_cast<int32_t>((static_cast<uint32_t>(b) << 16) | static_cast<uint32_t>(p)));
    }
    n += parts;
  }
  if (n > INT32_MAX) return -PA_ERR_INVALID;
  if (n > cap || items == nullptr) return static_cast<int32_t>(n);
  int64_t k = 0;
  for (int64_t s = part_blocks; s >= 0; --s)
    for (int32_t v : by_size[static_cast<size_t>(s)]) items[k++] = v;
  return static_cast<int32_t>(n);
}
