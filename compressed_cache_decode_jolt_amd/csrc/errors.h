// Error reporting shared by the library's C entry points.
#pragma once
#include <exception>
#include <new>
#include <stdexcept>

#include "jolt.h"

namespace jolt {

// Records the message returned by jolt_last_error() and returns st.
jolt_status set_error(jolt_status st, const char *fmt, ...);

// Runs body() and turns a C++ exception into an error status, so that none
// crosses the C ABI: host allocation failures (and containers asked for more
// than they can hold) become JOLT_E_OOM, anything else JOLT_E_INVALID with
// the exception's message.
template <typename F>
jolt_status guarded(const char *what, F &&body) {
  try {
    return body();
  } catch (const std::bad_alloc &) {
    return set_error(JOLT_E_OOM, "%s: host allocation failed", what);
  } catch (const std::length_error &) {
    return set_error(JOLT_E_OOM, "%s: host allocation too large", what);
  } catch (const std::exception &e) {
    return set_error(JOLT_E_INVALID, "%s: %s", what, e.what());
  } catch (...) {
    return set_error(JOLT_E_INVALID, "%s: unexpected error", what);
  }
}

}  // namespace jolt
