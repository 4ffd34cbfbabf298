// Host-side checks of device-call inputs that the kernels cannot make
// cheaply themselves.
#include <algorithm>
#include <cstdint>
#include <utility>
#include <vector>

#include "pagedkv.h"
#include "status.h"

using pkv::fail;

// Two tokens of one cache write naming the same slot would leave that slot
// holding whichever landed last; the slot mapping of the Paged KV Cache
// Engine ("NeuralOps v1.3.4") gives every token its own slot, and the
// allocator never repeats one.
extern "C" int paged_kv_check_slots(const int32_t *slots, int32_t T, int64_t num_slots,
                                    int32_t *first_dup) {
  if (T < 0 || num_slots < 0) return fail(PKV_EINVAL, "T and num_slots must be >= 0");
  if (T > 0 && !slots) return fail(PKV_EINVAL, "slots is NULL");
  if (first_dup) *first_dup = -1;
  std::vector<std::pair<int32_t, int32_t>> seen;  // (slot, token)
  seen.reserve(T);
  for (int32_t t = 0; t < T; ++t)
    if (slots[t] >= 0 && slots[t] < num_slots) seen.emplace_back(slots[t], t);
  std::sort(seen.begin(), seen.end());
  int32_t dup = -1;
  for (size_t i = 1; i < seen.size(); ++i)
    if (seen[i].first == seen[i - 1].first && (dup < 0 || seen[i].second < dup))
      dup = seen[i].second;  // the later of the two tokens, earliest such
  if (dup < 0) return PKV_OK;
  if (first_dup) *first_dup = dup;
  return fail(PKV_EINVAL, "token %d writes slot %d, which an earlier token of the same write "
              "also names", dup, slots[dup]);
}
