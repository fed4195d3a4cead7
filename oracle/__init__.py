"""CPU oracle for the AWQ scale search — test infrastructure only (tests, smoke check,
benchmark CPU baseline). The GPU library never imports it."""
