// Launch-size limit shared by the host entry points.
#pragma once

#include <cstdint>

namespace pkv {

// Largest workgroup count of one launch.  A dispatch's work-item count
// (workgroups x threads per workgroup) must fit 32 bits, and no launch here
// uses more than 256 threads per workgroup.
constexpr int64_t kMaxGridGroups = (int64_t(1) << 24) - 1;

// Largest row count of one bucket launch: the rows are the third grid
// dimension, whose size HIP bounds by 65535 workgroups.
constexpr int64_t kMaxBucketRows = 65535;

}  // namespace pkv
