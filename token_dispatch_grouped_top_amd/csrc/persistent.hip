// persistent.hip -- placeholder until the persistent pipeline lands.
#include "persistent.h"

namespace mok {

size_t persistent_ws_bytes(int64_t total_windows) {
  return static_cast<size_t>(total_windows > 0 ? total_windows : 1) * 64 + 4096;
}

mok_status launch_persistent(const PersistentArgs&, hipStream_t) { return MOK_ERR_UNSUPPORTED; }

}  // namespace mok
