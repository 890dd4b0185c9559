// Rolling z-score of a scalar series (host only).
//
// The training log of the llm.c GPT-2 1.5B run (dszhyy.com post, setup
// section) prints next to the loss and the gradient norm of every step
// their z-score against the recent steps ("nanz" while there is no history
// yet), and the run was later restarted with flags that skip an update
// whose loss or norm z-score exceeds 5 (400B-token run section).  This is that
// detector: z of a new value against the mean and (population) standard
// deviation of the last `window` finite values, in double precision, each
// recomputed from the window itself so that no running sum drifts.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <limits>
#include <new>
#include <vector>

#include "../../include/gpt2.h"

int gpt2_internal_fail(int code, const char* msg);

struct gpt2_zscore {
  std::vector<double> ring;  // the last `window` finite values, oldest at `head` once full
  int head = 0;
  int count = 0;
};

extern "C" {

int gpt2_zscore_create(int window, gpt2_zscore** out) {
  if (!out) return gpt2_internal_fail(GPT2_EINVAL, "NULL output pointer");
  *out = nullptr;
  if (window < 2 || window > 65536)
    return gpt2_internal_fail(GPT2_EINVAL, "z-score window must be in [2, 65536]");
  gpt2_zscore* zs = new (std::nothrow) gpt2_zscore;
  if (!zs) return gpt2_internal_fail(GPT2_EINVAL, "out of host memory");
  zs->ring.assign((size_t)window, 0.0);
  *out = zs;
  return GPT2_OK;
}

int gpt2_zscore_update(gpt2_zscore* zs, double x, double* z_out) {
  if (!zs) return gpt2_internal_fail(GPT2_EINVAL, "NULL detector");
  const int w = (int)zs->ring.size();
  double z = std::numeric_limits<double>::quiet_NaN();
  if (zs->count == w && std::isfinite(x)) {
    // sums taken oldest first (the full ring's oldest value is at head), so
    // that a detector restored by gpt2_zscore_set_state gives the same bits
    double mean = 0.0;
    for (int i = 0; i < w; ++i) mean += zs->ring[(size_t)((zs->head + i) % w)];
    mean /= w;
    double var = 0.0;
    for (int i = 0; i < w; ++i) {
      const double d = zs->ring[(size_t)((zs->head + i) % w)] - mean;
      var += d * d;
    }
    const double sd = std::sqrt(var / w);
    if (sd > 0.0) z = (x - mean) / sd;
  }
  if (std::isfinite(x)) {
    zs->ring[(size_t)zs->head] = x;
    zs->head = (zs->head + 1) % w;
    if (zs->count < w) ++zs->count;
  }
  if (z_out) *z_out = z;
  return GPT2_OK;
}

int gpt2_zscore_get_state(const gpt2_zscore* zs, double* values, int cap, int* window,
                          int* count) {
  if (!zs) return gpt2_internal_fail(GPT2_EINVAL, "NULL detector");
  const int w = (int)zs->ring.size();
  if (window) *window = w;
  if (count) *count = zs->count;
  if (!values) return GPT2_OK;
  if (cap < zs->count) return gpt2_internal_fail(GPT2_EINVAL, "values holds fewer than count");
  // oldest first: before the window fills, slots 0 .. count-1 in order;
  // once full, from `head` around the ring
  const int start = zs->count == w ? zs->head : 0;
  for (int i = 0; i < zs->count; ++i) values[i] = zs->ring[(size_t)((start + i) % w)];
  return GPT2_OK;
}

int gpt2_zscore_set_state(gpt2_zscore* zs, const double* values, int count) {
  if (!zs) return gpt2_internal_fail(GPT2_EINVAL, "NULL detector");
  const int w = (int)zs->ring.size();
  if (count < 0 || count > w || (count > 0 && !values))
    return gpt2_internal_fail(GPT2_EINVAL, "count must be in [0, window] with values given");
  for (int i = 0; i < count; ++i)
    if (!std::isfinite(values[i]))
      return gpt2_internal_fail(GPT2_EINVAL, "a window holds finite values only");
  std::fill(zs->ring.begin(), zs->ring.end(), 0.0);
  for (int i = 0; i < count; ++i) zs->ring[(size_t)i] = values[i];
  zs->count = count;
  zs->head = count % w;
  return GPT2_OK;
}

int gpt2_zscore_destroy(gpt2_zscore* zs) {
  delete zs;
  return GPT2_OK;
}

}  // extern "C"
